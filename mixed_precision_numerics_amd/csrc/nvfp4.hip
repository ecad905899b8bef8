// NVFP4 two-level quantizer for the weight-gradient GEMM inputs (gfx950).
//
// Page "Pretraining Large Language Models with NVFP4" (gist.science):
// section 2.1 (E2M1 elements in blocks of 16 with an E4M3 scale per block and
// an FP32 scale per tensor), section 2.2 item 2 (16x16 random Hadamard
// transform on the weight-gradient inputs), item 3 (16x16 two-dimensional
// blocks for weights), item 4 (stochastic rounding of gradients).
//
// The quantized operand op = x or x^T has shape [R, K]; blocks, the RHT and
// the packing run along K.  Two passes over x:
//   pass 1  z = RHT(op) per 16-chunk; A = max|z| (bit-pattern max) -> atomic max
//   final   enc = fl32(2688 / A) if A is finite and > 0 else 1; dec = fl32(1/enc)
//   pass 2  per block: b = max|z|; s = E4M3_sat(fl32(fl32(b / 6) * enc));
//           S = decode(s); y = fl32(z * fl32(enc / S)); code = E2M1(y)
//           (nearest-even, or stochastic with the Philox4x32-10 word of the
//           element's row-major index idx = r*K + k; u = (w >> 8) * 2^-24);
//           S == 0 (or not a number) gives code 0.
// RHT order (fixed so that results are bit-reproducible): multiply by the
// signs (exact), butterflies (a, b) -> (a + b, a - b) at strides 1, 2, 4, 8,
// each rounded to FP32, then * 0.25.
//
// Work layout: a block stages a 64 (op rows) x 256 (K) tile of op in LDS as
// FP32 (row pitch 257 words, so both the transposing stores and the row reads
// spread over the banks); thread t takes op row t % 64 and the four 16-chunks
// 4*(t/64) .. 4*(t/64)+3, i.e. writes 32 contiguous bytes of codes and 4
// scale bytes.  For 16x16 blocks the 16 rows of a block are 16 consecutive
// lanes and the block amax is a 16-lane shuffle reduction.
#include "common.hpp"
#include "formats.hpp"

namespace amp {
namespace {

constexpr int kT = 256;          // threads
constexpr int kRows = 64;        // op rows per tile
constexpr int kK = 256;          // K per tile
constexpr int kPitch = kK + 1;   // LDS row pitch in floats

template <int XT>
__device__ __forceinline__ float ld_x(const void* x, int64_t i) {
  if constexpr (XT == AMP_BF16) return bf16_to_f32(static_cast<const uint16_t*>(x)[i]);
  else return static_cast<const float*>(x)[i];
}

// Stage op[r0 : r0+64, k0 : k0+256] into lds[r][k] (zero outside [R, K]).
template <int XT, bool TRANS>
__device__ __forceinline__ void stage_tile(const void* x, int64_t ldx, int64_t R, int64_t K,
                                           int64_t r0, int64_t k0, float* lds) {
  const int t = threadIdx.x;
  if constexpr (!TRANS) {
    // x rows are op rows: coalesced along k
#pragma unroll 4
    for (int e = t; e < kRows * kK; e += kT) {
      const int r = e / kK, k = e % kK;
      const int64_t gr = r0 + r, gk = k0 + k;
      lds[r * kPitch + k] = (gr < R && gk < K) ? ld_x<XT>(x, gr * ldx + gk) : 0.0f;
    }
  } else {
    // x rows are K: coalesced along the op rows, stored transposed
#pragma unroll 4
    for (int e = t; e < kRows * kK; e += kT) {
      const int k = e / kRows, r = e % kRows;
      const int64_t gr = r0 + r, gk = k0 + k;
      lds[r * kPitch + k] = (gr < R && gk < K) ? ld_x<XT>(x, gk * ldx + gr) : 0.0f;
    }
  }
}

__device__ __forceinline__ void rht16(float (&z)[16], uint32_t sign_bits) {
#pragma unroll
  for (int j = 0; j < 16; ++j) z[j] = ((sign_bits >> j) & 1u) ? -z[j] : z[j];
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int blk = 0; blk < 16; blk += 2 * h) {
#pragma unroll
      for (int i = blk; i < blk + h; ++i) {
        const float a = z[i], b = z[i + h];
        z[i] = a + b;
        z[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) z[j] = z[j] * 0.25f;
}

__device__ __forceinline__ uint32_t rht_signs(uint64_t seed) {
  const ctr4 w = philox4x32_10(ctr4{0u, 0u, 1u, 0u}, static_cast<uint32_t>(seed),
                               static_cast<uint32_t>(seed >> 32));
  return w.x & 0xffffu;
}

__global__ void zero_amax(float* d_tensor) {
  if (threadIdx.x == 0) d_tensor[0] = 0.0f;
}

__global__ void finalize_enc(float* d_tensor) {
  if (threadIdx.x != 0) return;
  const uint32_t a = fbits(d_tensor[0]);
  float enc = 1.0f;
  if (a < 0x7f800000u && a != 0u) enc = 2688.0f / bitsf(a);
  d_tensor[1] = enc;
  d_tensor[2] = 1.0f / enc;
}

// PASS2 = false: tensor amax only.
template <int XT, bool TRANS, bool PASS2, bool BLOCK2D, bool RHT, bool SR>
__global__ __launch_bounds__(kT) void nvfp4_kernel(const void* __restrict__ x, int64_t ldx,
                                                   int64_t R, int64_t K, uint64_t rht_seed,
                                                   uint64_t sr_seed, uint8_t* __restrict__ q,
                                                   uint8_t* __restrict__ scales,
                                                   float* __restrict__ d_tensor) {
  __shared__ float lds[kRows * kPitch];
  __shared__ uint32_t red[kT / kWave];
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kRows;
  const int64_t k0 = static_cast<int64_t>(blockIdx.x) * kK;
  stage_tile<XT, TRANS>(x, ldx, R, K, r0, k0, lds);
  __syncthreads();

  const int t = threadIdx.x;
  const int r = t % kRows;
  const int g = t / kRows;                 // chunk group: chunks 4g .. 4g+3
  const int64_t gr = r0 + r;
  const uint32_t sign_bits = RHT ? rht_signs(rht_seed) : 0u;
  const float enc = PASS2 ? d_tensor[1] : 1.0f;
  uint32_t am = 0;
  uint32_t qwords[8];
  uint32_t sbytes = 0;

#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const int kc = (4 * g + cc) * 16;      // k offset in the tile
    const int64_t gk = k0 + kc;
    float z[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = lds[r * kPitch + kc + j];
    if constexpr (RHT) rht16(z, sign_bits);
    uint32_t bmax = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t a = fbits(z[j]) & 0x7fffffffu;
      bmax = bmax > a ? bmax : a;
    }
    if constexpr (!PASS2) {
      am = am > bmax ? am : bmax;
      continue;
    } else {
      if constexpr (BLOCK2D) {
        // rows r0+16q .. +15 of this chunk are 16 consecutive lanes
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(bmax), off, kWave));
          bmax = bmax > o ? bmax : o;
        }
      }
      const float b = bitsf(bmax);
      const uint32_t scode = f32_to_e4m3((b / 6.0f) * enc);
      const float S = e4m3_to_f32(scode);
      const bool live = S > 0.0f;
      const float mult = live ? enc / S : 0.0f;
      uint32_t codes[16];
      if constexpr (SR) {
        // Philox word (idx & 3) of counter idx >> 2, idx = gr * K + gk + j
        const uint64_t idx0 = static_cast<uint64_t>(gr) * static_cast<uint64_t>(K) +
                              static_cast<uint64_t>(gk);
#pragma unroll
        for (int quad = 0; quad < 4; ++quad) {
          const uint64_t blk = (idx0 >> 2) + quad;
          const ctr4 w = philox4x32_10(
              ctr4{static_cast<uint32_t>(blk), static_cast<uint32_t>(blk >> 32), 0u, 0u},
              static_cast<uint32_t>(sr_seed), static_cast<uint32_t>(sr_seed >> 32));
          const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) codes[4 * quad + e] = e2m1_sr(z[4 * quad + e] * mult, ww[e]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) codes[j] = e2m1_rne(z[j] * mult);
      }
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t c = live ? codes[j] : 0u;
        w0 |= c << (4 * j);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t c = live ? codes[8 + j] : 0u;
        w1 |= c << (4 * j);
      }
      qwords[2 * cc] = w0;
      qwords[2 * cc + 1] = w1;
      sbytes |= scode << (8 * cc);
    }
  }

  if constexpr (!PASS2) {
    am = block_max_u32<kT>(am, red);
    if (t == 0 && am != 0) amax_update(d_tensor, am);
  } else {
    if (gr < R) {
      const int64_t kq = (k0 + 64 * g) / 2;           // byte offset of this thread's codes
      uint8_t* dst = q + gr * (K / 2) + kq;
      const int64_t kvalid = K - (k0 + 64 * g);        // elements of this group inside K
      if (kvalid >= 64) {
        *reinterpret_cast<u32x4*>(dst) = u32x4{qwords[0], qwords[1], qwords[2], qwords[3]};
        *reinterpret_cast<u32x4*>(dst + 16) = u32x4{qwords[4], qwords[5], qwords[6], qwords[7]};
      } else {
        for (int c = 0; c < 4; ++c)
          if (16 * c < kvalid) {
            *reinterpret_cast<uint32_t*>(dst + 8 * c) = qwords[2 * c];
            *reinterpret_cast<uint32_t*>(dst + 8 * c + 4) = qwords[2 * c + 1];
          }
      }
      const int64_t kb = (k0 + 64 * g) / 16;           // first block index along K
      if constexpr (BLOCK2D) {
        if ((gr & 15) == 0) {
          uint8_t* sd = scales + (gr / 16) * (K / 16) + kb;
          for (int c = 0; c < 4; ++c)
            if (16 * c < kvalid) sd[c] = static_cast<uint8_t>(sbytes >> (8 * c));
        }
      } else {
        uint8_t* sd = scales + gr * (K / 16) + kb;
        if (kvalid >= 64) {
          *reinterpret_cast<uint32_t*>(sd) = sbytes;
        } else {
          for (int c = 0; c < 4; ++c)
            if (16 * c < kvalid) sd[c] = static_cast<uint8_t>(sbytes >> (8 * c));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Vector path (16-byte aligned rows).  No LDS staging: a lane owns a "cell"
// of CW op rows x one 16-chunk along K, fetched with sixteen 16-byte loads
// (CW = 8 for BF16, 4 for FP32), and runs the RHT, the block amax and the
// encoding in registers, one op row at a time.
//   transposed operand (x rows are K): lane = cg + 8*kc -> op rows CW*cg..,
//     chunk kc; one load instruction reads 8 x rows x 128 contiguous bytes.
//   plain operand (x rows are op rows): lane = rg + G*kc (G = 16/CW) -> op
//     rows CW*rg.., chunk kc; consecutive lanes walk along K.
// In both, the CW-row groups of one 16-row block are G adjacent lanes, so a
// 16x16 block amax is a G-lane xor-shuffle reduction.  A wave tile is
// TILE_R op rows x TILE_K; a row of a tile writes 128 (transposed) or 256
// (plain) contiguous code bytes.  WIDE (the transposed operand's amax pass,
// which has no blocks to encode): all 64 lanes across op rows, so that one
// load instruction reads 1 KiB of one x row.
template <int XT, bool TRANS, bool WIDE = false>
struct VecGeom {
  static constexpr int kESize = XT == AMP_BF16 ? 2 : 4;
  static constexpr int kCW = 16 / kESize;          // op rows per lane
  static constexpr int kG = 16 / kCW;              // lanes per 16-row block
  static constexpr int kLR = TRANS ? (WIDE ? kWave : 8) : kG;   // lanes across op rows
  static constexpr int kLK = kWave / kLR;          // lanes across K
  static constexpr int kTileR = kLR * kCW;
  static constexpr int kSubK = 16 * kLK;
  static constexpr int kNSub = TRANS ? 2 : 1;
  static constexpr int kTileK = kSubK * kNSub;
};

template <int XT, bool TRANS>
__device__ __forceinline__ void load_cell(const uint8_t* __restrict__ xb, int64_t ldb, int64_t gr,
                                          int64_t gk, bool valid, u32x4 (&raw)[16]) {
  using Gm = VecGeom<XT, TRANS>;
#pragma unroll
  for (int j = 0; j < 16; ++j) raw[j] = u32x4{0u, 0u, 0u, 0u};
  if (!valid) return;
  if constexpr (TRANS) {
    const uint8_t* p = xb + gk * ldb + gr * Gm::kESize;
#pragma unroll
    for (int j = 0; j < 16; ++j) raw[j] = *reinterpret_cast<const u32x4*>(p + j * ldb);
  } else {
    const uint8_t* p = xb + gr * ldb + gk * Gm::kESize;
    constexpr int kPerRow = Gm::kESize;            // 16 elements = kESize x 16 bytes
#pragma unroll
    for (int i = 0; i < Gm::kCW; ++i)
#pragma unroll
      for (int h = 0; h < kPerRow; ++h)
        raw[i * kPerRow + h] = *reinterpret_cast<const u32x4*>(p + i * ldb + 16 * h);
  }
}

// Element (op row i of the cell, K offset j of the chunk).
template <int XT, bool TRANS>
__device__ __forceinline__ float cell_elem(const u32x4 (&raw)[16], int i, int j) {
  if constexpr (TRANS) {
    if constexpr (XT == AMP_BF16) {
      const uint32_t w = raw[j][i >> 1];
      return bitsf((i & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
      return bitsf(raw[j][i]);
    }
  } else {
    if constexpr (XT == AMP_BF16) {
      const uint32_t w = raw[2 * i + (j >> 3)][(j & 7) >> 1];
      return bitsf((j & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
      return bitsf(raw[4 * i + (j >> 2)][j & 3]);
    }
  }
}

template <int XT, bool TRANS, bool RHT>
__device__ __forceinline__ uint32_t row_chunk(const u32x4 (&raw)[16], int i, uint32_t sign_bits,
                                              float (&z)[16]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) z[j] = cell_elem<XT, TRANS>(raw, i, j);
  if constexpr (RHT) rht16(z, sign_bits);
  uint32_t bmax = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t a = fbits(z[j]) & 0x7fffffffu;
    bmax = bmax > a ? bmax : a;
  }
  return bmax;
}

// Philox4x32-10 on the four counters blk0 .. blk0+3 (high words from blk),
// side by side: the four independent chains fill the multiplier's latency.
// The rounds run two per loop iteration, so that the state words alternate
// between two register sets instead of being copied back every round.
__device__ __forceinline__ void philox_x4(uint64_t blk0, uint64_t seed, uint32_t (&w)[16]) {
  uint32_t x[4], y[4], z[4], v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint64_t blk = blk0 + q;
    x[q] = static_cast<uint32_t>(blk);
    y[q] = static_cast<uint32_t>(blk >> 32);
    z[q] = 0u;
    v[q] = 0u;
  }
  uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
#pragma unroll 2
  for (int r = 0; r < 10; ++r) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * x[q];
      const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * z[q];
      x[q] = xor3(static_cast<uint32_t>(p1 >> 32), y[q], k0);
      y[q] = static_cast<uint32_t>(p1);
      z[q] = xor3(static_cast<uint32_t>(p0 >> 32), v[q], k1);
      v[q] = static_cast<uint32_t>(p0);
    }
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    w[4 * q] = x[q];
    w[4 * q + 1] = y[q];
    w[4 * q + 2] = z[q];
    w[4 * q + 3] = v[q];
  }
}

template <bool SR>
__device__ __forceinline__ u32x2 encode_chunk(const float (&z)[16], float mult, bool live,
                                              uint64_t idx0, uint64_t sr_seed) {
  uint32_t codes[16];
  if constexpr (SR) {
    // word (idx & 3) of the Philox block idx >> 2, idx = idx0 + j
    uint32_t w[16];
    philox_x4(idx0 >> 2, sr_seed, w);
#pragma unroll
    for (int j = 0; j < 16; ++j) codes[j] = e2m1_sr(z[j] * mult, w[j]);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) codes[j] = e2m1_rne(z[j] * mult);
  }
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    w0 |= codes[j] << (4 * j);
    w1 |= codes[8 + j] << (4 * j);
  }
  return live ? u32x2{w0, w1} : u32x2{0u, 0u};
}

// PASS2 = false: tensor amax only.
template <int XT, bool TRANS, bool PASS2, bool BLOCK2D, bool RHT, bool SR>
__global__ __launch_bounds__(kT) void nvfp4_vec_kernel(
    const uint8_t* __restrict__ xb, int64_t ldb, int64_t R, int64_t K, int64_t tiles_r,
    int64_t tiles_k, uint64_t rht_seed, uint64_t sr_seed, uint8_t* __restrict__ q,
    uint8_t* __restrict__ scales, float* __restrict__ d_tensor) {
  using Gm = VecGeom<XT, TRANS, TRANS && !PASS2>;
  __shared__ uint32_t red[kT / kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int lr = lane % Gm::kLR;
  const int lk = lane / Gm::kLR;
  const uint32_t sign_bits = RHT ? rht_signs(rht_seed) : 0u;
  const float enc = PASS2 ? d_tensor[1] : 1.0f;
  const int64_t ntiles = tiles_r * tiles_k;
  const int64_t wstride = static_cast<int64_t>(gridDim.x) * (kT / kWave);
  uint32_t am = 0;
  for (int64_t w = static_cast<int64_t>(blockIdx.x) * (kT / kWave) + threadIdx.x / kWave;
       w < ntiles; w += wstride) {
    // neighbouring waves read neighbouring bytes of the same x rows
    const int64_t tr = TRANS ? w % tiles_r : w / tiles_k;
    const int64_t tk = TRANS ? w / tiles_r : w % tiles_k;
    const int64_t gr = tr * Gm::kTileR + Gm::kCW * lr;
// one K-subtile of the tile; the stochastic-rounding pass keeps both
    // subtiles' loads in flight, the others run them one after the other
    // (fewer live registers, more waves per SIMD: measured faster for them)
    auto subtile = [&](int sub) __attribute__((always_inline)) {
      const int64_t gk = tk * Gm::kTileK + sub * Gm::kSubK + 16 * lk;
      const bool valid = gr < R && gk < K;
      u32x4 raw[16];
      load_cell<XT, TRANS>(xb, ldb, gr, gk, valid, raw);
      if constexpr (!PASS2) {
#pragma unroll
        for (int i = 0; i < Gm::kCW; ++i) {
          float z[16];
          const uint32_t b = row_chunk<XT, TRANS, RHT>(raw, i, sign_bits, z);
          am = am > b ? am : b;
        }
      } else if constexpr (BLOCK2D) {
        // block amax over the CW rows here and the G-1 neighbouring lanes,
        // then a second RHT per row for the encoding
        uint32_t bmax = 0;
#pragma unroll
        for (int i = 0; i < Gm::kCW; ++i) {
          float z[16];
          const uint32_t b = row_chunk<XT, TRANS, RHT>(raw, i, sign_bits, z);
          bmax = bmax > b ? bmax : b;
        }
#pragma unroll
        for (int off = 1; off < Gm::kG; off <<= 1) {
          const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(bmax), off, kWave));
          bmax = bmax > o ? bmax : o;
        }
        const uint32_t scode = f32_to_e4m3((bitsf(bmax) / 6.0f) * enc);
        const float S = e4m3_to_f32(scode);
        const bool live = S > 0.0f;
        const float mult = live ? enc / S : 0.0f;
#pragma unroll
        for (int i = 0; i < Gm::kCW; ++i) {
          float z[16];
          (void)row_chunk<XT, TRANS, RHT>(raw, i, sign_bits, z);
          const uint64_t idx0 = static_cast<uint64_t>(gr + i) * static_cast<uint64_t>(K) +
                                static_cast<uint64_t>(gk);
          const u32x2 cw = encode_chunk<SR>(z, mult, live, idx0, sr_seed);
          if (valid) *reinterpret_cast<u32x2*>(q + (gr + i) * (K / 2) + gk / 2) = cw;
        }
        if (valid && (lr % Gm::kG) == 0)
          scales[(gr / 16) * (K / 16) + gk / 16] = static_cast<uint8_t>(scode);
      } else {
#pragma unroll
        for (int i = 0; i < Gm::kCW; ++i) {
          float z[16];
          const uint32_t bmax = row_chunk<XT, TRANS, RHT>(raw, i, sign_bits, z);
          const uint32_t scode = f32_to_e4m3((bitsf(bmax) / 6.0f) * enc);
          const float S = e4m3_to_f32(scode);
          const bool live = S > 0.0f;
          const float mult = live ? enc / S : 0.0f;
          const uint64_t idx0 = static_cast<uint64_t>(gr + i) * static_cast<uint64_t>(K) +
                                static_cast<uint64_t>(gk);
          const u32x2 cw = encode_chunk<SR>(z, mult, live, idx0, sr_seed);
          if (valid) {
            *reinterpret_cast<u32x2*>(q + (gr + i) * (K / 2) + gk / 2) = cw;
            scales[(gr + i) * (K / 16) + gk / 16] = static_cast<uint8_t>(scode);
          }
        }
      }
    };
    if constexpr (PASS2 && SR) {
#pragma unroll
      for (int sub = 0; sub < Gm::kNSub; ++sub) subtile(sub);
    } else {
#pragma unroll 1
      for (int sub = 0; sub < Gm::kNSub; ++sub) subtile(sub);
    }
  }
  if constexpr (!PASS2) {
    am = block_max_u32<kT>(am, red);
    if (threadIdx.x == 0 && am != 0)
      amax_update(d_tensor, am);
  }
}

template <int XT, bool TRANS, bool BLOCK2D, bool RHT, bool SR>
hipError_t run_vec(const void* x, int64_t ldx, int64_t R, int64_t K, uint64_t rs, uint64_t ss,
                   uint8_t* q, uint8_t* sc, float* dt, hipStream_t s) {
  using Gm = VecGeom<XT, TRANS>;                    // encode pass
  using Ga = VecGeom<XT, TRANS, TRANS>;             // amax pass
  const int64_t tiles_r = (R + Gm::kTileR - 1) / Gm::kTileR;
  const int64_t tiles_k = (K + Gm::kTileK - 1) / Gm::kTileK;
  const int64_t atiles_r = (R + Ga::kTileR - 1) / Ga::kTileR;
  const int64_t atiles_k = (K + Ga::kTileK - 1) / Ga::kTileK;
  auto* amax_pass = nvfp4_vec_kernel<XT, TRANS, false, BLOCK2D, RHT, SR>;
  auto* encode_pass = nvfp4_vec_kernel<XT, TRANS, true, BLOCK2D, RHT, SR>;
  // one wave per tile up to 2^16 waves (a longer loop per wave beyond that)
  auto grid = [](int64_t ntiles) {
    int64_t blocks = (ntiles + kT / kWave - 1) / (kT / kWave);
    return static_cast<unsigned>(blocks > 16384 ? 16384 : blocks);
  };
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  const int64_t ldb = ldx * Gm::kESize;
  zero_amax<<<1, 64, 0, s>>>(dt);
  amax_pass<<<grid(atiles_r * atiles_k), kT, 0, s>>>(xb, ldb, R, K, atiles_r, atiles_k, rs, ss, q, sc, dt);
  finalize_enc<<<1, 64, 0, s>>>(dt);
  encode_pass<<<grid(tiles_r * tiles_k), kT, 0, s>>>(xb, ldb, R, K, tiles_r, tiles_k, rs, ss, q, sc, dt);
  return hipGetLastError();
}

template <int XT, bool TRANS, bool BLOCK2D, bool RHT, bool SR>
hipError_t run(const void* x, int64_t ldx, int64_t R, int64_t K, uint64_t rs, uint64_t ss,
               uint8_t* q, uint8_t* sc, float* dt, hipStream_t s) {
  // 16-byte vector loads need 16-byte aligned rows; codes are stored 8 bytes
  // at a time
  const int64_t esize = XT == AMP_BF16 ? 2 : 4;
  if (aligned(x, 16) && (ldx * esize) % 16 == 0 && aligned(q, 8))
    return run_vec<XT, TRANS, BLOCK2D, RHT, SR>(x, ldx, R, K, rs, ss, q, sc, dt, s);
  const dim3 grid(static_cast<unsigned>((K + kK - 1) / kK), static_cast<unsigned>((R + kRows - 1) / kRows));
  zero_amax<<<1, 64, 0, s>>>(dt);
  nvfp4_kernel<XT, TRANS, false, BLOCK2D, RHT, SR><<<grid, kT, 0, s>>>(x, ldx, R, K, rs, ss, q, sc, dt);
  finalize_enc<<<1, 64, 0, s>>>(dt);
  nvfp4_kernel<XT, TRANS, true, BLOCK2D, RHT, SR><<<grid, kT, 0, s>>>(x, ldx, R, K, rs, ss, q, sc, dt);
  return hipGetLastError();
}

template <int XT, bool TRANS>
hipError_t run_opts(int block2d, int rht, int sr, const void* x, int64_t ldx, int64_t R, int64_t K,
                    uint64_t rs, uint64_t ss, uint8_t* q, uint8_t* sc, float* dt, hipStream_t s) {
#define AMP_NV(B, H, S) return run<XT, TRANS, B, H, S>(x, ldx, R, K, rs, ss, q, sc, dt, s)
  if (block2d) {
    if (rht) { if (sr) AMP_NV(true, true, true); AMP_NV(true, true, false); }
    if (sr) AMP_NV(true, false, true);
    AMP_NV(true, false, false);
  }
  if (rht) { if (sr) AMP_NV(false, true, true); AMP_NV(false, true, false); }
  if (sr) AMP_NV(false, false, true);
  AMP_NV(false, false, false);
#undef AMP_NV
}

}  // namespace

hipError_t launch_nvfp4_quantize(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                                 int transpose, int block2d, int rht, uint64_t rht_seed, int rnd,
                                 uint64_t sr_seed, uint8_t* q, uint8_t* scales, float* d_tensor,
                                 hipStream_t s) {
  const int64_t R = transpose ? cols : rows, K = transpose ? rows : cols;
  const int sr = rnd == AMP_ROUND_SR;
  if (R == 0 || K == 0) {
    zero_amax<<<1, 64, 0, s>>>(d_tensor);
    finalize_enc<<<1, 64, 0, s>>>(d_tensor);
    return hipGetLastError();
  }
  if (xt == AMP_BF16) {
    if (transpose) return run_opts<AMP_BF16, true>(block2d, rht, sr, x, ldx, R, K, rht_seed, sr_seed, q, scales, d_tensor, s);
    return run_opts<AMP_BF16, false>(block2d, rht, sr, x, ldx, R, K, rht_seed, sr_seed, q, scales, d_tensor, s);
  }
  if (transpose) return run_opts<AMP_F32, true>(block2d, rht, sr, x, ldx, R, K, rht_seed, sr_seed, q, scales, d_tensor, s);
  return run_opts<AMP_F32, false>(block2d, rht, sr, x, ldx, R, K, rht_seed, sr_seed, q, scales, d_tensor, s);
}

}  // namespace amp
