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
          for (int e = 0; e < 4; ++e) {
            const float u = static_cast<float>(ww[e] >> 8) * 5.9604644775390625e-8f;
            codes[4 * quad + e] = e2m1_sr(z[4 * quad + e] * mult, u);
          }
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
    if (t == 0 && am != 0) atomicMax(reinterpret_cast<unsigned int*>(d_tensor), canon_amax(am));
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

template <int XT, bool TRANS, bool BLOCK2D, bool RHT, bool SR>
hipError_t run(const void* x, int64_t ldx, int64_t R, int64_t K, uint64_t rs, uint64_t ss,
               uint8_t* q, uint8_t* sc, float* dt, hipStream_t s) {
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
