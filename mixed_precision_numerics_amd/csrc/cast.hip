// Scaled down-cast with amax capture (gfx950).
//
// What is computed: page "FP8 혼합 정밀도 LLM 학습" (hwlabs), sections
// "FP8이 어려운 이유" (a per-tensor scale brings the tensor into the FP8 range,
// values are clipped to [-448, 448]) and "Delayed Scaling 동작 원리" (each
// step records the tensor's amax; with the scale known in advance the tensor
// is read once); page "혼합 정밀도 학습" (itwiki), section "FP16 학습 루프"
// (16-bit copies are made from the FP32 parameters just before use).
//
//   y = round(fl32(x * scale)),  amax = max(amax, max|x|)  (bit-pattern max)
//
// Two kernels, both HBM-bound:
//  * cast_flat: contiguous tensors; each block converts contiguous ranges of
//    2048 8-element vectors with non-temporal 16-byte loads, four in flight
//    per thread, and one atomic max per block.
//  * cast_tile: strided tensors and the optional transposed copy (the FP8
//    dgrad / wgrad operands).  A 256-thread block owns a 128x128 tile; each
//    thread converts an 8x8 sub-block, writes its row-major codes directly and
//    its transposed codes into LDS, from where the block writes the transposed
//    tile with coalesced 16-byte stores.
#include "common.hpp"
#include "formats.hpp"

namespace amp {
namespace {

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

template <int XT>
__device__ __forceinline__ float load_one(const void* p, int64_t i) {
  if constexpr (XT == AMP_F32) return static_cast<const float*>(p)[i];
  else if constexpr (XT == AMP_BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return f16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

// Load 8 consecutive elements (16-byte aligned); NT marks the loads
// non-temporal (data read once by a streaming pass).
template <int XT, bool NT = false>
__device__ __forceinline__ void load8(const void* p, int64_t i, float (&v)[8]) {
  if constexpr (XT == AMP_F32) {
    const f32x4* q = reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
    f32x4 a, b;
    if constexpr (NT) { a = __builtin_nontemporal_load(q); b = __builtin_nontemporal_load(q + 1); }
    else { a = q[0]; b = q[1]; }
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const u32x4* q = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p) + i);
    const u32x4 w = NT ? __builtin_nontemporal_load(q) : *q;
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (XT == AMP_BF16) {
        v[2 * k] = bitsf(ww[k] << 16);
        v[2 * k + 1] = bitsf(ww[k] & 0xffff0000u);
      } else {
        v[2 * k] = f16_to_f32(ww[k] & 0xffffu);
        v[2 * k + 1] = f16_to_f32(ww[k] >> 16);
      }
    }
  }
}

template <int YT>
__device__ __forceinline__ uint32_t to_code(float t) {
  if constexpr (YT == AMP_F16) return f32_to_f16(t);
  else if constexpr (YT == AMP_BF16) return f32_to_bf16(t);
  else if constexpr (YT == AMP_E4M3) return f32_to_e4m3(t);
  else return f32_to_e5m2(t);
}

template <int YT>
struct CodeT { using type = uint16_t; };
template <> struct CodeT<AMP_E4M3> { using type = uint8_t; };
template <> struct CodeT<AMP_E5M2> { using type = uint8_t; };

// Store 8 codes at y + i (8- or 16-byte aligned); NT as for load8.
template <int YT, bool NT = false>
__device__ __forceinline__ void store8(void* y, int64_t i, const uint32_t (&c)[8]) {
  if constexpr (sizeof(typename CodeT<YT>::type) == 1) {
    u32x2 w;
    w.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    w.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    u32x2* q = reinterpret_cast<u32x2*>(static_cast<uint8_t*>(y) + i);
    if constexpr (NT) __builtin_nontemporal_store(w, q);
    else *q = w;
  } else {
    u32x4 w;
    w.x = c[0] | (c[1] << 16); w.y = c[2] | (c[3] << 16);
    w.z = c[4] | (c[5] << 16); w.w = c[6] | (c[7] << 16);
    u32x4* q = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + i);
    if constexpr (NT) __builtin_nontemporal_store(w, q);
    else *q = w;
  }
}

// Store 4 codes at y + i (4- or 8-byte aligned); NT as for load8.
template <int YT, bool NT = false>
__device__ __forceinline__ void store4(void* y, int64_t i, const uint32_t* c) {
  if constexpr (sizeof(typename CodeT<YT>::type) == 1) {
    const uint32_t w = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    uint32_t* q = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(y) + i);
    if constexpr (NT) __builtin_nontemporal_store(w, q);
    else *q = w;
  } else {
    u32x2 w;
    w.x = c[0] | (c[1] << 16); w.y = c[2] | (c[3] << 16);
    u32x2* q = reinterpret_cast<u32x2*>(static_cast<uint16_t*>(y) + i);
    if constexpr (NT) __builtin_nontemporal_store(w, q);
    else *q = w;
  }
}

template <int YT>
__device__ __forceinline__ void store_one(void* y, int64_t i, uint32_t c) {
  static_cast<typename CodeT<YT>::type*>(y)[i] = static_cast<typename CodeT<YT>::type>(c);
}

// Saturating (FP8) outputs: elements whose scaled value lies beyond the
// format's largest magnitude are clipped; the optional counter records them
// (inf included, NaN not).
template <int YT> struct SatMax { static constexpr bool on = false; static constexpr float v = 0.0f; };
template <> struct SatMax<AMP_E4M3> { static constexpr bool on = true; static constexpr float v = 448.0f; };
template <> struct SatMax<AMP_E5M2> { static constexpr bool on = true; static constexpr float v = 57344.0f; };

// Wave sum of per-lane counts, one 64-bit atomic add per wave (all lanes call).
__device__ __forceinline__ void add_sat(uint32_t n, unsigned long long* d_sat) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) n += static_cast<uint32_t>(__shfl_xor(static_cast<int>(n), off, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0 && n != 0) atomicAdd(d_sat, static_cast<unsigned long long>(n));
}

constexpr int kFlatThreads = 256;

constexpr int kFlatUnroll = 4;
constexpr int64_t kFlatChunk = 2048;           // 8-element vectors per range (32 KiB of BF16)
constexpr int64_t kFlatMaxBlocks = 256 * 64;   // one amax atomic per work-group

// Vector path: the input is cut into ranges of kFlatChunk vectors; work-group
// b converts ranges b, b + G, b + 2G, ... (G work-groups), each thread with
// four 16-byte loads in flight, all accesses non-temporal (the source is read
// once and the codes are consumed by a later kernel); the last work-group also
// converts the n % 8 trailing elements.  For 2^31 BF16 -> E4M3 codes this ran
// at 5.70 TB/s in a probe of the same access shape, against 5.45 for one
// 16384-vector range per work-group and 4.9 for a grid-stride loop over single
// vectors.  FP32 input: a wave's 8 vectors of an unrolled step are its 512
// consecutive elements, lane l taking elements 4l .. 4l+3 and 256+4l ..
// 256+4l+3, so that every load and store instruction covers one contiguous
// span (with 8 consecutive elements per lane the two loads of an instruction
// pair each touched every other 16 bytes of a 2 KiB span).  Scalar path: a
// grid-stride loop.
template <int XT, int YT, bool VEC, bool SAT>
__global__ __launch_bounds__(kFlatThreads) void cast_flat(const void* __restrict__ x,
                                                          void* __restrict__ y, int64_t n,
                                                          const float* __restrict__ d_scale,
                                                          float* __restrict__ d_amax,
                                                          unsigned long long* __restrict__ d_sat) {
  __shared__ uint32_t red[kFlatThreads / kWave];
  const bool SCALE = d_scale != nullptr, AMAX = d_amax != nullptr;
  uint32_t ns = 0;
  const float scale = SCALE ? *d_scale : 1.0f;
  uint32_t am = 0;
  auto encode1 = [&](int64_t i, float v) __attribute__((always_inline)) {
    if (AMAX) { const uint32_t a = fbits(v) & 0x7fffffffu; am = am > a ? am : a; }
    const float t = SCALE ? v * scale : v;
    if constexpr (SAT) ns += fabsf(t) > SatMax<YT>::v;
    store_one<YT>(y, i, to_code<YT>(t));
  };
  if constexpr (VEC) {
    const int64_t nv = n / 8;
    auto encode8 = [&](int64_t j, const float (&v)[8]) __attribute__((always_inline)) {
      uint32_t c[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (AMAX) { const uint32_t a = fbits(v[k]) & 0x7fffffffu; am = am > a ? am : a; }
        const float t = SCALE ? v[k] * scale : v[k];
        if constexpr (SAT) ns += fabsf(t) > SatMax<YT>::v;
        c[k] = to_code<YT>(t);
      }
      store8<YT, true>(y, j * 8, c);
    };
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kFlatChunk;
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    for (int64_t b0 = static_cast<int64_t>(blockIdx.x) * kFlatChunk; b0 < nv; b0 += stride) {
      const int64_t b1 = b0 + kFlatChunk < nv ? b0 + kFlatChunk : nv;
      int64_t jb = b0;   // the block's first vector of the step
      for (; jb + kFlatUnroll * kFlatThreads <= b1; jb += kFlatUnroll * kFlatThreads) {
        float v[kFlatUnroll][8];
        if constexpr (XT == AMP_F32) {
          // e: this lane's first element of step u; the second four are 256 on
#pragma unroll
          for (int u = 0; u < kFlatUnroll; ++u) {
            const f32x4* q = reinterpret_cast<const f32x4*>(
                static_cast<const float*>(x) + (jb + u * kFlatThreads) * 8 + 512 * wv + 4 * lane);
            const f32x4 a = __builtin_nontemporal_load(q), b = __builtin_nontemporal_load(q + 64);
            v[u][0] = a.x; v[u][1] = a.y; v[u][2] = a.z; v[u][3] = a.w;
            v[u][4] = b.x; v[u][5] = b.y; v[u][6] = b.z; v[u][7] = b.w;
          }
#pragma unroll
          for (int u = 0; u < kFlatUnroll; ++u) {
            uint32_t c[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              if (AMAX) { const uint32_t a = fbits(v[u][k]) & 0x7fffffffu; am = am > a ? am : a; }
              const float t = SCALE ? v[u][k] * scale : v[u][k];
              if constexpr (SAT) ns += fabsf(t) > SatMax<YT>::v;
              c[k] = to_code<YT>(t);
            }
            const int64_t e = (jb + u * kFlatThreads) * 8 + 512 * wv + 4 * lane;
            store4<YT, true>(y, e, c);
            store4<YT, true>(y, e + 256, c + 4);
          }
        } else {
          const int64_t j = jb + threadIdx.x;
#pragma unroll
          for (int u = 0; u < kFlatUnroll; ++u) load8<XT, true>(x, (j + u * kFlatThreads) * 8, v[u]);
#pragma unroll
          for (int u = 0; u < kFlatUnroll; ++u) encode8(j + u * kFlatThreads, v[u]);
        }
      }
      for (int64_t j = jb + threadIdx.x; j < b1; j += kFlatThreads) {
        float v[8];
        load8<XT, true>(x, j * 8, v);
        encode8(j, v);
      }
    }
    if (blockIdx.x == gridDim.x - 1)
      for (int64_t i = nv * 8 + threadIdx.x; i < n; i += kFlatThreads) encode1(i, load_one<XT>(x, i));
  } else {
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kFlatThreads + threadIdx.x;
    const int64_t nthr = static_cast<int64_t>(gridDim.x) * kFlatThreads;
    for (int64_t i = tid; i < n; i += nthr) encode1(i, load_one<XT>(x, i));
  }
  if constexpr (SAT) add_sat(ns, d_sat);
  if (AMAX) {
    am = block_max_u32<kFlatThreads>(am, red);
    if (threadIdx.x == 0 && am != 0)
      amax_update(d_amax, am);
  }
}

constexpr int kTile = 128;
constexpr int kTileThreads = 256;

// 128x128 tile per block.  Thread t owns rows r0..r0+7 and columns c0..c0+7
// with c0 = 8*(t % 16), r0 = 8*(t / 16).  FULL: the tile is inside the tensor
// and every access is 16-byte aligned (checked on the host).
__device__ __forceinline__ int swz8(int c) { return (2 * (c >> 4)) & 14; }

// VEC: 0 element loads; 1 16-byte accesses, edge tiles element by element;
// 2 16-byte accesses and every tile full (no edge code in the kernel, which
// keeps the edge path's registers out of its allocation).
template <int XT, int YT, bool WY, bool WYT, int VEC, bool SAT>
__global__ __launch_bounds__(kTileThreads) void cast_tile(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    void* __restrict__ y, int64_t ldy, void* __restrict__ y_t, int64_t ldy_t,
    const float* __restrict__ d_scale, float* __restrict__ d_amax,
    unsigned long long* __restrict__ d_sat) {
  using Code = typename CodeT<YT>::type;
  constexpr int kPitch = kTile + 16 / static_cast<int>(sizeof(Code));  // row pitch in codes
  __shared__ __align__(16) Code lds[WYT ? kTile * kPitch : 1];
  __shared__ uint32_t red[kTileThreads / kWave];

  const bool SCALE = d_scale != nullptr, AMAX = d_amax != nullptr;
  uint32_t ns = 0;
  const float scale = SCALE ? *d_scale : 1.0f;
  const int64_t r_base = static_cast<int64_t>(blockIdx.y) * kTile;
  const int64_t c_base = static_cast<int64_t>(blockIdx.x) * kTile;
  const int t = threadIdx.x;
  const int c0 = 8 * (t % 16), r0 = 8 * (t / 16);
  // a thread's 8 columns: c0 .. c0+7, or for FP32 input 4c .. 4c+3 and
  // 64+4c .. 64+4c+3 (c = t % 16), so that each 16-byte load instruction of
  // a wave covers 256 contiguous bytes of a row (eight consecutive FP32
  // columns per lane made each of its two loads touch every other 16 bytes)
  constexpr bool kSplit = XT == AMP_F32;
  auto col = [&](int j) { return kSplit ? (j < 4 ? 4 * (t % 16) + j : 64 + 4 * (t % 16) + (j - 4)) : c0 + j; };
  const bool full = VEC == 2 || (VEC == 1 && (r_base + kTile <= rows) && (c_base + kTile <= cols));
  uint32_t am = 0;
  // 16-bit codes are kept one per register; 8-bit ones four per register
  // (row i's codes 4q .. 4q+3 in pk[i][q]), which cuts the live registers
  // from 64 to 16 and lets more blocks share a CU
  constexpr bool kPack = sizeof(Code) == 1;
  uint32_t code[kPack ? 1 : 8][8];
  uint32_t pk[kPack ? 8 : 1][2];

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = r_base + r0 + i;
    const int64_t c = c_base + c0;
    float v[8];
    if (full) {
      if constexpr (kSplit) {
        const float* xr = static_cast<const float*>(x) + r * ldx + c_base;
        const f32x4 a = *reinterpret_cast<const f32x4*>(xr + col(0));
        const f32x4 b = *reinterpret_cast<const f32x4*>(xr + col(4));
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      } else {
        load8<XT>(x, r * ldx + c, v);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t cj = c_base + col(j);
        v[j] = (r < rows && cj < cols) ? load_one<XT>(x, r * ldx + cj) : 0.0f;
      }
    }
    uint32_t c8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (AMAX) { const uint32_t a = fbits(v[j]) & 0x7fffffffu; am = am > a ? am : a; }
      const float t = SCALE ? v[j] * scale : v[j];
      // padding outside the tensor is 0 and never counts
      if constexpr (SAT) ns += fabsf(t) > SatMax<YT>::v;
      c8[j] = to_code<YT>(t);
    }
    if constexpr (kPack) {
      pk[i][0] = c8[0] | (c8[1] << 8) | (c8[2] << 16) | (c8[3] << 24);
      pk[i][1] = c8[4] | (c8[5] << 8) | (c8[6] << 16) | (c8[7] << 24);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) code[i][j] = c8[j];
    }
    if constexpr (WY) {
      if (full) {
        if constexpr (kSplit) {
          store4<YT>(y, r * ldy + c_base + col(0), c8);
          store4<YT>(y, r * ldy + c_base + col(4), c8 + 4);
        } else {
          store8<YT>(y, r * ldy + c, c8);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int64_t cj = c_base + col(j);
          if (r < rows && cj < cols) store_one<YT>(y, r * ldy + cj, c8[j]);
        }
      }
    }
  }

  if constexpr (WYT) {
    // transposed 8x8 sub-block -> LDS rows col(j), columns r0..r0+7.  8-bit
    // codes: the 8-byte unit r0/8 of row c is stored at unit (r0/8) ^ sw(c),
    // sw(c) = 2*(c/16) mod 16 (even, so 16-byte pairs stay adjacent), which
    // spreads a wave's stores (rows 8 apart) and the row reads over the banks
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      Code* dst = lds + col(j) * kPitch + r0;
      if constexpr (kPack) {
        dst = lds + col(j) * kPitch + 8 * ((r0 / 8) ^ swz8(col(j)));
        // column j = byte j%4 of pk[i][j/4] for rows i = 0..7, gathered with
        // byte permutes (selector s < 4: byte s of the second operand, 4..7:
        // byte s-4 of the first, 12: zero)
        const int q = j >> 2;
        const uint32_t sel = static_cast<uint32_t>(j & 3) | (static_cast<uint32_t>((j & 3) + 4) << 8) | 0x0c0c0000u;
        const uint32_t t01 = __builtin_amdgcn_perm(pk[1][q], pk[0][q], sel);
        const uint32_t t23 = __builtin_amdgcn_perm(pk[3][q], pk[2][q], sel);
        const uint32_t t45 = __builtin_amdgcn_perm(pk[5][q], pk[4][q], sel);
        const uint32_t t67 = __builtin_amdgcn_perm(pk[7][q], pk[6][q], sel);
        uint2 w;
        w.x = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
        w.y = __builtin_amdgcn_perm(t67, t45, 0x05040100u);
        *reinterpret_cast<uint2*>(dst) = w;
      } else {
        uint4 w;
        w.x = code[0][j] | (code[1][j] << 16); w.y = code[2][j] | (code[3][j] << 16);
        w.z = code[4][j] | (code[5][j] << 16); w.w = code[6][j] | (code[7][j] << 16);
        *reinterpret_cast<uint4*>(dst) = w;
      }
    }
    __syncthreads();
    // y_t rows c_base + cc hold tile rows r_base .. r_base + 127
    constexpr int kPer = 16 / static_cast<int>(sizeof(Code));       // codes per 16 B
    constexpr int kChunksPerRow = kTile / kPer;
    constexpr int kIters = kTile * kChunksPerRow / kTileThreads;
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int idx = it * kTileThreads + t;
      const int cc = idx / kChunksPerRow;
      const int rr = (idx % kChunksPerRow) * kPer;
      const int64_t orow = c_base + cc;
      const int64_t ocol = r_base + rr;
      const Code* src = lds + cc * kPitch + rr;
      if constexpr (sizeof(Code) == 1) src = lds + cc * kPitch + 8 * ((rr / 8) ^ swz8(cc));
      if (full) {
        *reinterpret_cast<uint4*>(static_cast<Code*>(y_t) + orow * ldy_t + ocol) =
            *reinterpret_cast<const uint4*>(src);
      } else if (orow < cols) {
#pragma unroll
        for (int k = 0; k < kPer; ++k)
          if (ocol + k < rows) static_cast<Code*>(y_t)[orow * ldy_t + ocol + k] = src[k];
      }
    }
  }

  if constexpr (SAT) add_sat(ns, d_sat);
  if (AMAX) {
    am = block_max_u32<kTileThreads>(am, red);
    if (t == 0 && am != 0) amax_update(d_amax, am);
  }
}

template <int XT, int YT, bool SAT>
hipError_t dispatch_layout_t(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* y,
                             int64_t ldy, void* y_t, int64_t ldy_t, const float* d_scale,
                             float* d_amax, unsigned long long* d_sat, hipStream_t s) {
  const int xb = dtype_bytes(XT), yb = dtype_bytes(YT);
  if (y_t == nullptr && ldx == cols && ldy == cols) {
    const int64_t n = rows * cols;
    const bool vec = aligned(x, 16) && aligned(y, 8 * yb);
    int64_t blocks = vec ? (n / 8 + kFlatChunk - 1) / kFlatChunk : (n + kFlatThreads - 1) / kFlatThreads;
    if (blocks > kFlatMaxBlocks) blocks = kFlatMaxBlocks;
    if (blocks < 1) blocks = 1;
    if (vec)
      cast_flat<XT, YT, true, SAT><<<dim3(static_cast<unsigned>(blocks)), kFlatThreads, 0, s>>>(
          x, y, n, d_scale, d_amax, d_sat);
    else
      cast_flat<XT, YT, false, SAT><<<dim3(static_cast<unsigned>(blocks)), kFlatThreads, 0, s>>>(
          x, y, n, d_scale, d_amax, d_sat);
    return hipGetLastError();
  }
  // the vector path needs every row start 16-byte aligned for x and the outputs
  bool vec = aligned(x, 16) && (ldx * xb) % 16 == 0;
  if (y) vec = vec && aligned(y, 8 * yb) && (ldy * yb) % (8 * yb) == 0;
  if (y_t) vec = vec && aligned(y_t, 16) && (ldy_t * yb) % 16 == 0;
  const dim3 grid(static_cast<unsigned>((cols + kTile - 1) / kTile),
                  static_cast<unsigned>((rows + kTile - 1) / kTile));
  const int vk = !vec ? 0 : (rows % kTile == 0 && cols % kTile == 0 ? 2 : 1);
#define AMP_TILE(WY, WYT, V) \
  cast_tile<XT, YT, WY, WYT, V, SAT><<<grid, kTileThreads, 0, s>>>( \
      x, rows, cols, ldx, y, ldy, y_t, ldy_t, d_scale, d_amax, d_sat)
#define AMP_TILE_V(WY, WYT) \
  do { if (vk == 2) AMP_TILE(WY, WYT, 2); else if (vk == 1) AMP_TILE(WY, WYT, 1); else AMP_TILE(WY, WYT, 0); } while (0)
  if (y && y_t) AMP_TILE_V(true, true);
  else if (y)   AMP_TILE_V(true, false);
  else          AMP_TILE_V(false, true);
#undef AMP_TILE_V
#undef AMP_TILE
  return hipGetLastError();
}

// The saturation counter is a separate instantiation (FP8 outputs only), so
// the plain cast carries no counting code.
template <int XT, int YT>
hipError_t dispatch_layout(const void* x, int64_t rows, int64_t cols, int64_t ldx, void* y,
                           int64_t ldy, void* y_t, int64_t ldy_t, const float* d_scale,
                           float* d_amax, unsigned long long* d_sat, hipStream_t s) {
  if constexpr (SatMax<YT>::on) {
    if (d_sat)
      return dispatch_layout_t<XT, YT, true>(x, rows, cols, ldx, y, ldy, y_t, ldy_t, d_scale,
                                             d_amax, d_sat, s);
  }
  return dispatch_layout_t<XT, YT, false>(x, rows, cols, ldx, y, ldy, y_t, ldy_t, d_scale, d_amax,
                                          nullptr, s);
}

template <int XT>
hipError_t dispatch_out(int yt, const void* x, int64_t rows, int64_t cols, int64_t ldx, void* y,
                        int64_t ldy, void* y_t, int64_t ldy_t, const float* d_scale,
                        float* d_amax, unsigned long long* d_sat, hipStream_t s) {
  switch (yt) {
    case AMP_F16: return dispatch_layout<XT, AMP_F16>(x, rows, cols, ldx, y, ldy, y_t, ldy_t, d_scale, d_amax, d_sat, s);
    case AMP_BF16: return dispatch_layout<XT, AMP_BF16>(x, rows, cols, ldx, y, ldy, y_t, ldy_t, d_scale, d_amax, d_sat, s);
    case AMP_E4M3: return dispatch_layout<XT, AMP_E4M3>(x, rows, cols, ldx, y, ldy, y_t, ldy_t, d_scale, d_amax, d_sat, s);
    default: return dispatch_layout<XT, AMP_E5M2>(x, rows, cols, ldx, y, ldy, y_t, ldy_t, d_scale, d_amax, d_sat, s);
  }
}


// ------------------------------------------------- current scaling ---
// Page hwlabs, section "Delayed Scaling 동작 원리": current (just-in-time)
// scaling reads the tensor once for its amax and once more for the cast.

// amax (FP32 bit-max of |x|) of a [rows, cols] tensor with row stride ldx.
template <int XT, bool VEC>
__global__ __launch_bounds__(kFlatThreads) void amax_kernel(const void* __restrict__ x,
                                                           int64_t rows, int64_t cols,
                                                           int64_t ldx, float* __restrict__ d_amax) {
  __shared__ uint32_t red[kFlatThreads / kWave];
  uint32_t am = 0;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kFlatThreads + threadIdx.x;
  const int64_t nthr = static_cast<int64_t>(gridDim.x) * kFlatThreads;
  const int64_t n = rows * cols;
  auto take = [&](float v) {
    const uint32_t a = fbits(v) & 0x7fffffffu;
    am = am > a ? am : a;
  };
  if constexpr (VEC && XT == AMP_F32) {   // 16 bytes (4 elements) per lane: one contiguous span per load
    const int64_t n4 = n / 4;
    const f32x4* x4 = static_cast<const f32x4*>(x);
    for (int64_t j = tid; j < n4; j += nthr) {
      const f32x4 v = x4[j];
      take(v.x); take(v.y); take(v.z); take(v.w);
    }
    for (int64_t i = n4 * 4 + tid; i < n; i += nthr) take(load_one<XT>(x, i));
  } else if constexpr (VEC) {       // contiguous rows (ldx == cols), 16-byte aligned
    const int64_t nv = n / 8;
    for (int64_t j = tid; j < nv; j += nthr) {
      float v[8];
      load8<XT>(x, j * 8, v);
#pragma unroll
      for (int k = 0; k < 8; ++k) take(v[k]);
    }
    for (int64_t i = nv * 8 + tid; i < n; i += nthr) take(load_one<XT>(x, i));
  } else {
    for (int64_t i = tid; i < n; i += nthr) {
      const int64_t r = i / cols;
      take(load_one<XT>(x, r * ldx + (i - r * cols)));
    }
  }
  am = block_max_u32<kFlatThreads>(am, red);
  if (threadIdx.x == 0 && am != 0)
    amax_update(d_amax, am);
}

__global__ void meta_zero_amax(amp_fp8_meta* mt) {
  if (threadIdx.x == 0) mt->amax_cur = 0.0f;
}

// scale = fp8_max / (margin * amax) in FP32; 1 for a zero or non-finite amax.
__global__ void current_scale_kernel(amp_fp8_meta* mt, float fp8_max, float margin) {
  if (threadIdx.x != 0) return;
  const uint32_t b = fbits(mt->amax_cur);
  float scale = 1.0f;
  if (b < 0x7f800000u && b != 0u) scale = fp8_max / (margin * bitsf(b));
  mt->scale = scale;
  mt->scale_inv = 1.0f / scale;
}


// ------------------------------------------- fine-grained (tile) scaling ---
// Page itwiki, section "FP8 혼합 정밀도": DeepSeek-V3 computes FP8 scales on
// the fly per 1x128 tile of activations and per 128x128 block of weights.
// Each tile is scaled as by current scaling: scale = fp8_max / amax(tile)
// in FP32 (1 for a zero or non-finite amax), y = round(fl32(x * scale)).
// One 256-thread block per 128x128 region of x with cast_tile's thread
// layout.  Row tiles (1x128 of x) scale the plain output q; column tiles
// (1x128 of x^T, i.e. 128x1 of x) scale the transposed output qt; in block
// mode the whole region shares one scale in both orientations.  scale_inv is
// stored K-block-major: s[(c / 128) * lds + r] (row tiles) or
// s[(c / 128) * lds + r / 128] (blocks), and st likewise with rows and
// columns exchanged.

// Max over the 16 lanes of a DPP row (row_ror 8, 4, 2, 1).
__device__ __forceinline__ uint32_t max16(uint32_t v) {
  uint32_t o;
  o = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xf, 0xf, false));
  v = v > o ? v : o;
  o = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x124, 0xf, 0xf, false));
  v = v > o ? v : o;
  o = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x122, 0xf, 0xf, false));
  v = v > o ? v : o;
  o = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x121, 0xf, 0xf, false));
  return v > o ? v : o;
}

// Current-scaling scale of one tile from its |x| bit-pattern maximum.
__device__ __forceinline__ float tile_scale(uint32_t amax_bits, float fp8_max) {
  return (amax_bits == 0u || amax_bits >= 0x7f800000u) ? 1.0f : fp8_max / bitsf(amax_bits);
}

// VEC as for cast_tile.
template <int XT, int YT, bool BLOCK, bool WQ, bool WQT, int VEC>
__global__ __launch_bounds__(kTileThreads) void bw_quant_tile(
    const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t lds,
    uint8_t* __restrict__ qt, int64_t ldqt, float* __restrict__ st, int64_t ldst) {
  constexpr int kPitch = kTile + 16;
  constexpr bool kCols = WQT && !BLOCK;              // column tiles need a cross-wave max
  __shared__ __align__(16) uint8_t tl[WQT ? kTile * kPitch : 1];
  __shared__ uint32_t cpart[kCols ? 16 : 1][kCols ? kTile : 1];
  __shared__ float cscale[kCols ? kTile : 1];
  __shared__ uint32_t red[kTileThreads / kWave];
  __shared__ float bscale;
  constexpr float kMax = YT == AMP_E4M3 ? 448.0f : 57344.0f;

  const int64_t r_base = static_cast<int64_t>(blockIdx.y) * kTile;
  const int64_t c_base = static_cast<int64_t>(blockIdx.x) * kTile;
  const int t = threadIdx.x;
  const int c0 = 8 * (t % 16), r0 = 8 * (t / 16);
  const bool full = VEC == 2 || (VEC == 1 && (r_base + kTile <= rows) && (c_base + kTile <= cols));
  // 16-bit inputs stay packed (two per register, widened where used), which
  // halves the registers the 8x8 sub-block holds across the block barriers
  constexpr bool kPacked = XT != AMP_F32;
  uint32_t w16[kPacked ? 8 : 1][4];
  float v32[kPacked ? 1 : 8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = r_base + r0 + i, c = c_base + c0;
    if constexpr (kPacked) {
      if (full) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + r * ldx + c);
        w16[i][0] = w.x; w16[i][1] = w.y; w16[i][2] = w.z; w16[i][3] = w.w;
      } else {
        const uint16_t* xs = static_cast<const uint16_t*>(x);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = (r < rows && c + 2 * q < cols) ? xs[r * ldx + c + 2 * q] : 0u;
          const uint32_t hi = (r < rows && c + 2 * q + 1 < cols) ? xs[r * ldx + c + 2 * q + 1] : 0u;
          w16[i][q] = lo | (hi << 16);
        }
      }
    } else {
      if (full) {
        load8<XT>(x, r * ldx + c, v32[i]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          v32[i][j] = (r < rows && c + j < cols) ? load_one<XT>(x, r * ldx + c + j) : 0.0f;
      }
    }
  }
  // an empty asm that claims to change the packed words: the compiler then
  // widens them again where the column codes need them instead of keeping
  // all 64 widened values live across the column-scale barriers
  auto repack = [&]() __attribute__((always_inline)) {
    if constexpr (kPacked) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(w16[i][q]));
    }
  };
  auto val = [&](int i, int j) __attribute__((always_inline)) -> float {
    if constexpr (XT == AMP_BF16) {
      const uint32_t w = w16[i][j >> 1];
      return bitsf((j & 1) ? (w & 0xffff0000u) : (w << 16));
    } else if constexpr (XT == AMP_F16) {
      const uint32_t w = w16[i][j >> 1];
      return f16_to_f32((j & 1) ? (w >> 16) : (w & 0xffffu));
    } else {
      return v32[i][j];
    }
  };
  // |x| bit maxima of this thread's 8 rows and 8 columns (padding is 0).
  // 16-bit inputs: the magnitudes of a packed pair are compared as two
  // unsigned 16-bit halves (their order is the order of |x|, NaN above inf,
  // as for the FP32 patterns), and only each maximum is widened.
  uint32_t ra[8], ca[8];
  if constexpr (kPacked) {
    auto pmax = [](uint32_t a, uint32_t b) __attribute__((always_inline)) {
      return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                    __builtin_bit_cast(u16x2, b)));
    };
    auto wide = [](uint32_t h) __attribute__((always_inline)) -> uint32_t {
      if constexpr (XT == AMP_BF16) return h << 16;
      else return fbits(f16_to_f32(h));
    };
    uint32_t pc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pc[q] = w16[0][q] & 0x7fff7fffu;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t pr = w16[i][0] & 0x7fff7fffu;
#pragma unroll
      for (int q = 1; q < 4; ++q) pr = pmax(pr, w16[i][q] & 0x7fff7fffu);
      const uint32_t lo = pr & 0xffffu, hi = pr >> 16;
      ra[i] = wide(lo > hi ? lo : hi);
      if (i > 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) pc[q] = pmax(pc[q], w16[i][q] & 0x7fff7fffu);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ca[2 * q] = wide(pc[q] & 0xffffu);
      ca[2 * q + 1] = wide(pc[q] >> 16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) ca[j] = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ra[i] = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t a = fbits(val(i, j)) & 0x7fffffffu;
        ra[i] = ra[i] > a ? ra[i] : a;
        ca[j] = ca[j] > a ? ca[j] : a;
      }
    }
  }
  float cs[8];
  const int64_t kb_q = c_base / kTile, kb_t = r_base / kTile;
  // plain codes: written as soon as the row scales are known, so that the
  // row scales are dead while the column scales are formed
  auto encode_rows = [&](const float (&rs)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t r = r_base + r0 + i, c = c_base + c0;
      uint32_t code[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) code[j] = to_code<YT>(val(i, j) * rs[i]);
      if (full) {
        store8<YT>(q, r * ldq + c, code);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (r < rows && c + j < cols) q[r * ldq + c + j] = static_cast<uint8_t>(code[j]);
      }
    }
  };
  if constexpr (BLOCK) {
    uint32_t m = ra[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) m = m > ra[i] ? m : ra[i];
    m = block_max_u32<kTileThreads>(m, red);
    if (t == 0) {
      const float sc = tile_scale(m, kMax);
      bscale = sc;
      if (WQ) s[kb_q * lds + r_base / kTile] = 1.0f / sc;
      if (WQT) st[kb_t * ldst + c_base / kTile] = 1.0f / sc;
    }
    __syncthreads();
    float rs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) rs[i] = cs[i] = bscale;
    if constexpr (WQ) {
      encode_rows(rs);
      repack();
    }
  } else {
    if constexpr (WQ) {
      // the 16 threads of a row of the region are the 16 lanes of a DPP row
      float rs[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        rs[i] = tile_scale(max16(ra[i]), kMax);
        const int64_t r = r_base + r0 + i;
        if (t % 16 == 0 && r < rows) s[kb_q * lds + r] = 1.0f / rs[i];
      }
      encode_rows(rs);
      repack();
    }
    if constexpr (WQT) {
#pragma unroll
      for (int j = 0; j < 8; ++j) cpart[t / 16][c0 + j] = ca[j];
      __syncthreads();
      if (t < kTile) {
        uint32_t m = 0;
#pragma unroll
        for (int g = 0; g < 16; ++g) m = m > cpart[g][t] ? m : cpart[g][t];
        const float sc = tile_scale(m, kMax);
        cscale[t] = sc;
        if (c_base + t < cols) st[kb_t * ldst + c_base + t] = 1.0f / sc;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 8; ++j) cs[j] = cscale[c0 + j];
    }
  }
  if constexpr (WQT) {
    // column j of the sub-block -> LDS row c0 + j (cast_tile's swizzled layout)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t c8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c8[i] = to_code<YT>(val(i, j) * cs[j]);
      uint2 w;
      w.x = c8[0] | (c8[1] << 8) | (c8[2] << 16) | (c8[3] << 24);
      w.y = c8[4] | (c8[5] << 8) | (c8[6] << 16) | (c8[7] << 24);
      *reinterpret_cast<uint2*>(tl + (c0 + j) * kPitch + 8 * ((r0 / 8) ^ swz8(c0 + j))) = w;
    }
    __syncthreads();
    constexpr int kIters = kTile * (kTile / 16) / kTileThreads;
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int idx = it * kTileThreads + t;
      const int cc = idx / (kTile / 16);
      const int rr = (idx % (kTile / 16)) * 16;
      const int64_t orow = c_base + cc, ocol = r_base + rr;
      const uint8_t* src = tl + cc * kPitch + 8 * ((rr / 8) ^ swz8(cc));
      if (full) {
        *reinterpret_cast<uint4*>(qt + orow * ldqt + ocol) = *reinterpret_cast<const uint4*>(src);
      } else if (orow < cols) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if (ocol + k < rows) qt[orow * ldqt + ocol + k] = src[k];
      }
    }
  }
}

template <int XT, int YT>
hipError_t dispatch_bw(const void* x, int64_t rows, int64_t cols, int64_t ldx, int block,
                       uint8_t* q, int64_t ldq, float* s, int64_t lds, uint8_t* qt,
                       int64_t ldqt, float* st, int64_t ldst, hipStream_t hs) {
  const int xb = dtype_bytes(XT);
  bool vec = aligned(x, 16) && (ldx * xb) % 16 == 0;
  if (q) vec = vec && aligned(q, 8) && ldq % 8 == 0;
  if (qt) vec = vec && aligned(qt, 16) && ldqt % 16 == 0;
  const dim3 grid(static_cast<unsigned>((cols + kTile - 1) / kTile),
                  static_cast<unsigned>((rows + kTile - 1) / kTile));
  const int vk = !vec ? 0 : (rows % kTile == 0 && cols % kTile == 0 ? 2 : 1);
#define AMP_BW1(B, WQ, WQT, V)                                                                  \
  bw_quant_tile<XT, YT, B, WQ, WQT, V><<<grid, kTileThreads, 0, hs>>>(                         \
      x, rows, cols, ldx, q, ldq, s, lds, qt, ldqt, st, ldst)
#define AMP_BW(B, WQ, WQT)                                                                      \
  do {                                                                                         \
    if (vk == 2) AMP_BW1(B, WQ, WQT, 2);                                                       \
    else if (vk == 1) AMP_BW1(B, WQ, WQT, 1);                                                  \
    else AMP_BW1(B, WQ, WQT, 0);                                                               \
  } while (0)
  if (block) {
    if (q && qt) AMP_BW(true, true, true);
    else if (q) AMP_BW(true, true, false);
    else AMP_BW(true, false, true);
  } else {
    if (q && qt) AMP_BW(false, true, true);
    else if (q) AMP_BW(false, true, false);
    else AMP_BW(false, false, true);
  }
#undef AMP_BW
#undef AMP_BW1
  return hipGetLastError();
}

template <int XT>
hipError_t dispatch_bw_out(int yt, const void* x, int64_t rows, int64_t cols, int64_t ldx,
                           int block, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                           uint8_t* qt, int64_t ldqt, float* st, int64_t ldst, hipStream_t hs) {
  if (yt == AMP_E4M3)
    return dispatch_bw<XT, AMP_E4M3>(x, rows, cols, ldx, block, q, ldq, s, lds, qt, ldqt, st, ldst, hs);
  return dispatch_bw<XT, AMP_E5M2>(x, rows, cols, ldx, block, q, ldq, s, lds, qt, ldqt, st, ldst, hs);
}

}  // namespace

hipError_t launch_cast(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx, void* y,
                       int yt, int64_t ldy, void* y_t, int64_t ldy_t, const float* d_scale,
                       float* d_amax, unsigned long long* d_sat, hipStream_t s) {
  switch (xt) {
    case AMP_F32: return dispatch_out<AMP_F32>(yt, x, rows, cols, ldx, y, ldy, y_t, ldy_t, d_scale, d_amax, d_sat, s);
    case AMP_BF16: return dispatch_out<AMP_BF16>(yt, x, rows, cols, ldx, y, ldy, y_t, ldy_t, d_scale, d_amax, d_sat, s);
    default: return dispatch_out<AMP_F16>(yt, x, rows, cols, ldx, y, ldy, y_t, ldy_t, d_scale, d_amax, d_sat, s);
  }
}

hipError_t launch_cast_current(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                               void* y, int yt, int64_t ldy, void* y_t, int64_t ldy_t,
                               float fp8_max, float margin, amp_fp8_meta* meta, hipStream_t s) {
  meta_zero_amax<<<1, 64, 0, s>>>(meta);
  const bool vec = ldx == cols && aligned(x, 16);
  int64_t blocks = (rows * cols / (vec ? 8 : 1) + kFlatThreads - 1) / kFlatThreads;
  if (blocks > 256 * 16) blocks = 256 * 16;
  if (blocks < 1) blocks = 1;
  const dim3 grid(static_cast<unsigned>(blocks));
  float* am = &meta->amax_cur;
#define AMP_AMAX(T)                                                                     \
  if (vec) amax_kernel<T, true><<<grid, kFlatThreads, 0, s>>>(x, rows, cols, ldx, am);   \
  else amax_kernel<T, false><<<grid, kFlatThreads, 0, s>>>(x, rows, cols, ldx, am);
  switch (xt) {
    case AMP_F32: AMP_AMAX(AMP_F32) break;
    case AMP_BF16: AMP_AMAX(AMP_BF16) break;
    default: AMP_AMAX(AMP_F16) break;
  }
#undef AMP_AMAX
  current_scale_kernel<<<1, 64, 0, s>>>(meta, fp8_max, margin);
  if (hipError_t e = hipGetLastError()) return e;
  return launch_cast(x, xt, rows, cols, ldx, y, yt, ldy, y_t, ldy_t, &meta->scale, nullptr, nullptr, s);
}

hipError_t launch_quantize_blockwise(const void* x, int xt, int64_t rows, int64_t cols,
                                     int64_t ldx, int yt, int block, uint8_t* q, int64_t ldq,
                                     float* s, int64_t lds, uint8_t* qt, int64_t ldqt, float* st,
                                     int64_t ldst, hipStream_t hs) {
  switch (xt) {
    case AMP_F32: return dispatch_bw_out<AMP_F32>(yt, x, rows, cols, ldx, block, q, ldq, s, lds, qt, ldqt, st, ldst, hs);
    case AMP_BF16: return dispatch_bw_out<AMP_BF16>(yt, x, rows, cols, ldx, block, q, ldq, s, lds, qt, ldqt, st, ldst, hs);
    default: return dispatch_bw_out<AMP_F16>(yt, x, rows, cols, ldx, block, q, ldq, s, lds, qt, ldqt, st, ldst, hs);
  }
}

}  // namespace amp
