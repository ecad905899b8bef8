// Low-precision GEMM with FP32 accumulation on CDNA4 MFMA (gfx950).
//
// What is computed: page "혼합 정밀도 학습" (itwiki), section "FP32 누산과
// 연산별 정밀도" (16-bit products are accumulated in FP32 and the result is
// written in 16 bits); page "FP8 혼합 정밀도 LLM 학습" (hwlabs), section
// "GEMM 누적 정밀도 문제" (FP8 products, FP32 accumulation across partial
// sums, output cast); page "Mixed Precision Training/es" (marovi), section
// "La receta de precisión mixta".  For NVFP4 operands (page "Pretraining
// Large Language Models with NVFP4", section 2.1) each E2M1 element times its
// E4M3 block scale is exact in BF16 and in F16 (at most 6 significant bits,
// magnitudes 2^-10 .. 2688), so the operand is decoded exactly (to F16 per
// register fragment on the full-tile path, to BF16 on the way to LDS
// otherwise) and the tensor scales are applied in the epilogue.
//
//   C = out_cast( fl32(alphaA * alphaB) * sum_k op(A)[m,k] op(B)[k,n] )
//
// Kernel shape: one 256-thread block (4 waves, 2x2) per 256x256 output tile,
// each wave a 128x128 sub-tile of 4x4 MFMA 32x32 blocks with FP32
// accumulators.  K advances in steps whose LDS image is 128 bytes per row
// (64 16-bit or 128 8-bit elements) and two LDS stages alternate.
// Operand rows are stored K-contiguous in LDS with a 16-byte-chunk XOR
// swizzle (chunk ^ ((row ^ row >> 3) & 7)) so that both the MFMA fragment
// reads (32 consecutive rows, one chunk) and the transposed stores (rows 8
// apart) spread over the banks (measured: no bank conflicts).
//  * gemm_mfma_d2l: full tiles.  The next K-step is fetched with
//    direct-to-LDS loads (buffer_load ... lds, 16 B per lane, no VGPR
//    staging): lane l of each 1 KB load fetches the logical chunk that the
//    swizzle places at LDS byte 16*l.  8-bit and 4-bit operands stay in their
//    storage format in LDS and are widened per register fragment (FP8 ->
//    BF16, NVFP4 -> F16 x block scale) or fed to the block-scaled
//    instruction (MX); M/N-contiguous 16-bit operands are read with
//    transposing LDS reads.  The two stages are separate LDS objects that
//    the K loop names statically, two steps at a time, so the compiler sees
//    that one stage's loads and the other's fragment reads are independent;
//    kernels with transposing reads issue their loads as inline assembly
//    (see d2l16).
//  * gemm_mfma: any layout and ragged edges.  The next K-step is staged in
//    registers; operands whose contiguous dimension is M or N (dgrad's
//    weight, both wgrad operands) are loaded as 8x8 blocks and transposed in
//    registers with byte permutes before the LDS store.
// Tiles are ordered so that each XCD (own L2) works on a contiguous range of
// tiles, grouped 8 tile-rows at a time for L2 reuse.
#include <type_traits>

#include "common.hpp"
#include "formats.hpp"

namespace amp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256, kBN = 256, kThreads = 256;
constexpr int kRowBytes = 128;                       // LDS bytes per tile row per K-step
constexpr int kOperandBytes = 256 * kRowBytes;       // one operand, one stage

// How operands travel from HBM to the matrix cores.
enum Path : int {
  kP16 = 0,       // F16/BF16 operands, BF16/F16 MFMA 32x32x16, BK = 64
  kPF8Exact = 1,  // FP8 operands widened exactly to BF16 (gemm_mfma: on the way to LDS, BK = 64;
                  // gemm_mfma_d2l: FP8 in LDS, per register fragment, BK = 128), BF16 MFMA
  kPF8Native = 2, // FP8 operands in LDS, FP8 MFMA 32x32x64, BK = 128
  kPFP4 = 3,      // NVFP4 operands decoded (x block scale) to BF16, BF16 MFMA, BK = 64
  kPMX8 = 4,      // MX, FP8 elements + UE8M0 scale per 32: block-scaled MFMA, BK = 128
  kPMX4 = 5,      // MX, E2M1 elements + UE8M0 scale per 32: block-scaled MFMA, BK = 256
  kPFP4D = 6,     // NVFP4 codes in LDS, decoded per fragment to F16 x block scale, F16 MFMA, BK = 256
  kPMX8E = 7,     // MX, FP8 elements in LDS, widened per fragment to BF16 times the UE8M0 block
                  // scale (exact for scaled elements within BF16's range), BF16 MFMA, BK = 128
};

struct GemmArgs {
  const void* A;
  const void* B;
  void* C;
  int64_t M, N, K, lda, ldb, ldc;
  const float* alphaA;
  const float* alphaB;
  const uint8_t* sA;
  const uint8_t* sB;
  int64_t ldsA, ldsB;
  int s2dA, s2dB;
  int mx;          // block scales are UE8M0 per 32 (MX) instead of NVFP4's E4M3 per 16
};

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *static_cast<const u32x4*>(p); }

// The wave's index in its block.  It is the same for every lane, but the
// compiler cannot tell from threadIdx; taken through readfirstlane it lives
// in a scalar register, so buffer-load scalar offsets and LDS bases derived
// from it need no per-lane (waterfall) loop.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// 8x8 transpose of 16-bit elements held as 8 rows of 4 words.
__device__ __forceinline__ void transpose8x8_16(const u32x4 (&v)[8], u32x4 (&o)[8]) {
#pragma unroll
  for (int mm = 0; mm < 8; ++mm) {
    const uint32_t sel = (mm & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[mm][q] = __builtin_amdgcn_perm(v[2 * q + 1][mm >> 1], v[2 * q][mm >> 1], sel);
    }
  }
}

// FP8 (E4M3 or E5M2) -> BF16, exact: 2 values per conversion instruction.
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, float scale = 1.0f) {
  if constexpr (FMT == AMP_E4M3)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, scale, HI));
}

// A UE8M0 block scale 2^(c - 127) as the FP32 operand of the scaled
// conversions: code 0 is 2^-127 (an FP32 subnormal), 0xFF is NaN; both the
// value and its exponent field read as the same power of two.
__device__ __forceinline__ float e8m0_scale(uint32_t c) {
  return bitsf(c == 0u ? 0x00400000u : (c == 255u ? 0x7fc00000u : c << 23));
}

// Two E2M1 codes (byte SEL of w) times the block scale S -> two BF16.  The
// hardware conversion runs at scale 1 (exact); the product with the E4M3
// scale is formed in FP32, where it is exact (at most 6 significant bits,
// range 2^-10 .. 2688), and truncation to BF16 is therefore exact too.  (The
// conversion's own scale operand is not used: it only carries a power of two.)
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w, float S) {
  const uint32_t p = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
  const float lo = bitsf(p << 16) * S;
  const float hi = bitsf(p & 0xffff0000u) * S;
  return (fbits(lo) >> 16) | (fbits(hi) & 0xffff0000u);
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Eight E2M1 codes (one dword, lower k in the low nibble) times the E4M3
// block scale held twice in S -> eight F16 values (four dwords).  E2M1 to F16
// is exact (hardware conversion at scale 1) and so is the F16 product: at
// most 6 significant bits, magnitudes 2^-10 .. 2688, all normal in F16.
__device__ __forceinline__ u32x4 fp4x8_to_f16(uint32_t w, f16x2_t S) {
  u32x4 o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0)) * S);
  o[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1)) * S);
  o[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2)) * S);
  o[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3)) * S);
  return o;
}

// ---------------------------------------------------------------- loaders
// Each loader fetches one K-step of one operand (256 rows) into registers
// (`fetch`) and writes it to an LDS stage (`store`).  R: rows of the operand
// (M for A, N for B); ld: leading dimension in elements (bytes for FP4).

template <int ET, bool KC, int PATH>
struct Loader;

// 16-bit, K-contiguous: thread t owns chunk t%8 of rows t/8 + 32i.
template <int ET>
struct Loader<ET, true, kP16> {
  u32x4 v[8];
  template <bool CHECK>
  __device__ __forceinline__ void fetch(const void* X, int64_t ld, int64_t R, int64_t K,
                                        int64_t r0, int64_t k0, const uint8_t*, int64_t, int) {
    const int t = threadIdx.x;
    const int c = t & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t gr = r0 + (t >> 3) + 32 * i;
      const int64_t gk = k0 + 8 * c;
      v[i] = (!CHECK || (gr < R && gk < K)) ? ld16(static_cast<const uint16_t*>(X) + gr * ld + gk)
                                : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(lds + swz((t >> 3) + 32 * i, t & 7)) = v[i];
  }
};

// 16-bit, M/N-contiguous: thread t loads k rows 8g..8g+7 (g = t/32) of the
// 8-wide column chunk c = t%32, i.e. an 8x8 block, and transposes it.
template <int ET>
struct Loader<ET, false, kP16> {
  u32x4 v[8];
  template <bool CHECK>
  __device__ __forceinline__ void fetch(const void* X, int64_t ld, int64_t R, int64_t K,
                                        int64_t r0, int64_t k0, const uint8_t*, int64_t, int) {
    const int t = threadIdx.x;
    const int g = t >> 5, c = t & 31;
    const int64_t gr = r0 + 8 * c;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t gk = k0 + 8 * g + i;
      v[i] = (!CHECK || (gr < R && gk < K)) ? ld16(static_cast<const uint16_t*>(X) + gk * ld + gr)
                                : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int t = threadIdx.x;
    const int g = t >> 5, c = t & 31;
    u32x4 o[8];
    transpose8x8_16(v, o);
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) *reinterpret_cast<u32x4*>(lds + swz(8 * c + mm, g)) = o[mm];
  }
};

// FP8 -> BF16 (exact path), K-contiguous, BK = 64: thread t loads 16 FP8 of
// row t/4 + 64i at k offset 16*(t%4) and writes two 16-byte BF16 chunks.
template <int ET>
struct Loader<ET, true, kPF8Exact> {
  u32x4 v[4];
  template <bool CHECK>
  __device__ __forceinline__ void fetch(const void* X, int64_t ld, int64_t R, int64_t K,
                                        int64_t r0, int64_t k0, const uint8_t*, int64_t, int) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t gr = r0 + (t >> 2) + 64 * i;
      const int64_t gk = k0 + 16 * (t & 3);
      v[i] = (!CHECK || (gr < R && gk < K)) ? ld16(static_cast<const uint8_t*>(X) + gr * ld + gk)
                                : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (t >> 2) + 64 * i;
      u32x4 lo, hi;
      lo[0] = fp8x2_to_bf16x2<ET, false>(v[i][0]); lo[1] = fp8x2_to_bf16x2<ET, true>(v[i][0]);
      lo[2] = fp8x2_to_bf16x2<ET, false>(v[i][1]); lo[3] = fp8x2_to_bf16x2<ET, true>(v[i][1]);
      hi[0] = fp8x2_to_bf16x2<ET, false>(v[i][2]); hi[1] = fp8x2_to_bf16x2<ET, true>(v[i][2]);
      hi[2] = fp8x2_to_bf16x2<ET, false>(v[i][3]); hi[3] = fp8x2_to_bf16x2<ET, true>(v[i][3]);
      *reinterpret_cast<u32x4*>(lds + swz(row, 2 * (t & 3))) = lo;
      *reinterpret_cast<u32x4*>(lds + swz(row, 2 * (t & 3) + 1)) = hi;
    }
  }
};

// FP8 native, K-contiguous, BK = 128: same chunk map as the 16-bit loader.
template <int ET>
struct Loader<ET, true, kPF8Native> {
  u32x4 v[8];
  template <bool CHECK>
  __device__ __forceinline__ void fetch(const void* X, int64_t ld, int64_t R, int64_t K,
                                        int64_t r0, int64_t k0, const uint8_t*, int64_t, int) {
    const int t = threadIdx.x;
    const int c = t & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t gr = r0 + (t >> 3) + 32 * i;
      const int64_t gk = k0 + 16 * c;
      v[i] = (!CHECK || (gr < R && gk < K)) ? ld16(static_cast<const uint8_t*>(X) + gr * ld + gk)
                                : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(lds + swz((t >> 3) + 32 * i, t & 7)) = v[i];
  }
};

// NVFP4 -> BF16, K-contiguous, BK = 64: thread t loads 32 E2M1 codes (16 B) of
// row t/2 + 128i at k offset 32*(t%2) plus their two E4M3 block scales, and
// writes four 16-byte BF16 chunks of e2m1 * S.
template <int ET>
struct Loader<ET, true, kPFP4> {
  u32x4 v[2];
  uint32_t s[2];
  template <bool CHECK>
  __device__ __forceinline__ void fetch(const void* X, int64_t ld, int64_t R, int64_t K,
                                        int64_t r0, int64_t k0, const uint8_t* sc, int64_t lds_,
                                        int s2d) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t gr = r0 + (t >> 1) + 128 * i;
      const int64_t gk = k0 + 32 * (t & 1);
      const bool ok = !CHECK || (gr < R && gk < K);
      v[i] = ok ? ld16(static_cast<const uint8_t*>(X) + gr * ld + gk / 2) : u32x4{0, 0, 0, 0};
      const int64_t srow = s2d ? gr / 16 : gr;
      s[i] = ok ? *reinterpret_cast<const uint16_t*>(sc + srow * lds_ + gk / 16) : 0u;
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = (t >> 1) + 128 * i;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float S = e4m3_to_f32((s[i] >> (8 * half)) & 0xffu);
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const uint32_t w = v[i][2 * half + cc];
          u32x4 o;
          o[0] = fp4x2_to_bf16x2<0>(w, S);
          o[1] = fp4x2_to_bf16x2<1>(w, S);
          o[2] = fp4x2_to_bf16x2<2>(w, S);
          o[3] = fp4x2_to_bf16x2<3>(w, S);
          *reinterpret_cast<u32x4*>(lds + swz(row, 4 * (t & 1) + 2 * half + cc)) = o;
        }
      }
    }
  }
};

// ----------------------------------------------------------------- kernel

template <int CT>
__device__ __forceinline__ void store_c(void* C, int64_t idx, float x) {
  if constexpr (CT == AMP_F32) static_cast<float*>(C)[idx] = x;
  else if constexpr (CT == AMP_BF16) static_cast<uint16_t*>(C)[idx] = static_cast<uint16_t>(f32_to_bf16(x));
  else static_cast<uint16_t*>(C)[idx] = static_cast<uint16_t>(f32_to_f16(x));
}

template <int AT, int BT, bool A_KC, bool B_KC, int PATH, int CT, bool CHECK>
__global__ __launch_bounds__(kThreads, 1) void gemm_mfma(GemmArgs g) {
  __shared__ __align__(16) uint8_t smem[2][2][kOperandBytes];
  constexpr int BK = PATH == kPF8Native ? 128 : 64;

  // XCD-aware, L2-grouped tile order
  const int64_t nbm = (g.M + kBM - 1) / kBM, nbn = (g.N + kBN - 1) / kBN;
  const int64_t total = nbm * nbn;
  int64_t tile = blockIdx.x;
  if (total % 8 == 0) tile = (tile % 8) * (total / 8) + tile / 8;
  constexpr int64_t kGroup = 8;
  const int64_t group = tile / (kGroup * nbn);
  const int64_t first_m = group * kGroup;
  const int64_t gsz = nbm - first_m < kGroup ? nbm - first_m : kGroup;
  const int64_t in_group = tile % (kGroup * nbn);
  const int64_t tm = first_m + in_group % gsz;
  const int64_t tn = in_group / gsz;
  const int64_t m0 = tm * kBM, n0 = tn * kBN;

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  Loader<AT, A_KC, PATH> la;
  Loader<BT, B_KC, PATH> lb;
  const int64_t nk = (g.K + BK - 1) / BK;

  if (nk > 0) {
    la.template fetch<CHECK>(g.A, g.lda, g.M, g.K, m0, 0, g.sA, g.ldsA, g.s2dA);
    lb.template fetch<CHECK>(g.B, g.ldb, g.N, g.K, n0, 0, g.sB, g.ldsB, g.s2dB);
    la.store(smem[0][0]);
    lb.store(smem[0][1]);
    __syncthreads();
  }

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = static_cast<int>(kt & 1);
    if (kt + 1 < nk) {
      la.template fetch<CHECK>(g.A, g.lda, g.M, g.K, m0, (kt + 1) * BK, g.sA, g.ldsA, g.s2dA);
      lb.template fetch<CHECK>(g.B, g.ldb, g.N, g.K, n0, (kt + 1) * BK, g.sB, g.ldsB, g.s2dB);
    }
    const uint8_t* sa = smem[cur][0];
    const uint8_t* sb = smem[cur][1];
    if constexpr (PATH == kPF8Native) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        i32x8 af[4], bfr[4];
        const int ch = 4 * ks + 2 * (lane >> 5);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int row = wm * 128 + mb * 32 + (lane & 31);
          const u32x4 lo = *reinterpret_cast<const u32x4*>(sa + swz(row, ch));
          const u32x4 hi = *reinterpret_cast<const u32x4*>(sa + swz(row, ch + 1));
          af[mb] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int row = wn * 128 + nb * 32 + (lane & 31);
          const u32x4 lo = *reinterpret_cast<const u32x4*>(sb + swz(row, ch));
          const u32x4 hi = *reinterpret_cast<const u32x4*>(sb + swz(row, ch + 1));
          bfr[nb] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
        constexpr int fa = AT == AMP_E4M3 ? 0 : 1;
        constexpr int fb = BT == AMP_E4M3 ? 0 : 1;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[mb], bfr[nb], acc[mb][nb], fa, fb, 0, 127, 0, 127);
      }
    } else {
      u32x4 af[2][4], bfr[2][4];
      auto frag = [&](int ks, u32x4 (&a)[4], u32x4 (&b)[4]) {
        const int ch = 2 * ks + (lane >> 5);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          a[mb] = *reinterpret_cast<const u32x4*>(sa + swz(wm * 128 + mb * 32 + (lane & 31), ch));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          b[nb] = *reinterpret_cast<const u32x4*>(sb + swz(wn * 128 + nb * 32 + (lane & 31), ch));
      };
      frag(0, af[0], bfr[0]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks < 3) frag(ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            if constexpr (PATH == kP16 && AT == AMP_F16)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  __builtin_bit_cast(f16x8_t, af[ks & 1][mb]), __builtin_bit_cast(f16x8_t, bfr[ks & 1][nb]),
                  acc[mb][nb], 0, 0, 0);
            else
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8_t, af[ks & 1][mb]), __builtin_bit_cast(bf16x8_t, bfr[ks & 1][nb]),
                  acc[mb][nb], 0, 0, 0);
          }
      }
      // 64 MFMA, 32 DS reads (8 already issued), 16 VMEM loads
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    }
    if (kt + 1 < nk) {
      la.store(smem[cur ^ 1][0]);
      lb.store(smem[cur ^ 1][1]);
    }
    __syncthreads();
  }

  const float alpha = (g.alphaA ? *g.alphaA : 1.0f) * (g.alphaB ? *g.alphaB : 1.0f);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int64_t col = n0 + wn * 128 + nb * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < g.M && col < g.N) store_c<CT>(g.C, row * g.ldc + col, acc[mb][nb][r] * alpha);
      }
    }
}


// ------------------------------------------------------- direct-to-LDS NT
typedef __attribute__((address_space(3))) void lds_void;

// One 16-byte-per-lane direct-to-LDS load (64 lanes fill 1 KB at dst).  With
// ASM set it is written as inline assembly: the compiler then does not track
// it as a pending LDS write.  It has to be kept from tracking it where the
// transposing LDS reads follow: those reads carry no alias information, so
// the compiler would make the first of them wait for every load in flight,
// exposing the whole global-load latency in each K-step.  Every caller makes
// the loads land before their destination is read (s_waitcnt vmcnt(0), then
// a block barrier), which is the ordering the compiler would otherwise add.
template <bool ASM>
__device__ __forceinline__ void d2l16(__amdgpu_buffer_rsrc_t rsrc, uint8_t* dst, uint32_t voff,
                                      uint32_t soff) {
  if constexpr (ASM) {
    const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)dst));
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(m0)
                 : "memory");
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, voff, soff, 0, 0);
  }
}

// Wave w fills rows w*64 .. w*64+63 of a 256-row operand stage, 8 rows (1 KB)
// per buffer load; lane l writes LDS bytes 16*l of those 8 rows, i.e.
// physical chunk l%8 of row l/8, so it fetches the logical chunk that the
// swizzle maps there: p ^ (l/8) ^ i for the i-th load.  The buffer resource
// starts at the tile's first row; koff is the K-step's byte offset.
template <bool ASM = false>
__device__ __forceinline__ void d2l_stage(__amdgpu_buffer_rsrc_t rsrc, uint32_t ldb, uint32_t koff,
                                          uint8_t* stage) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const uint32_t vrow = static_cast<uint32_t>(w * 64 + lane / 8) * ldb;
  const uint32_t x = static_cast<uint32_t>(((lane & 7) ^ (lane >> 3)) & 7) << 4;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    d2l16<ASM>(rsrc, stage + (w * 64 + i * 8) * kRowBytes, vrow + (x ^ static_cast<uint32_t>(i << 4)),
               koff + static_cast<uint32_t>(8 * i) * ldb);
}

// M/N-contiguous 16-bit operand (rows of the global matrix are K): an LDS
// stage holds the step's 64 K-rows of the tile's 256 columns, 512 bytes per
// row, with 16-byte chunk c of K-row k stored at chunk c ^ 4*(k%4).  Wave w
// loads K-rows 16w .. 16w+15, two rows (1 KB) per buffer load: lane l writes
// physical chunk l%32 of row l/32.  rsrc starts at the step's first K-row.
// Always followed by transposing reads, so always the assembly form.
__device__ __forceinline__ void d2l_stage_mn(__amdgpu_buffer_rsrc_t rsrc, uint32_t ldb,
                                             uint8_t* stage) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int hr = lane >> 5;
  const uint32_t v0 = static_cast<uint32_t>(hr) * ldb;
  // row%4 = 2*(i&1) + hr
  const uint32_t ve = v0 + (static_cast<uint32_t>((lane & 31) ^ (4 * hr)) << 4);
  const uint32_t vo = v0 + (static_cast<uint32_t>((lane & 31) ^ (4 * (2 + hr))) << 4);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    d2l16<true>(rsrc, stage + (w * 16 + 2 * i) * 512, (i & 1) ? vo : ve,
                static_cast<uint32_t>(w * 16 + 2 * i) * ldb);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// MFMA 32x32x16 operand fragment (lane l: row l%32 of the 32-block, K
// 8*(l/32) .. +7) from an M/N-contiguous stage with two transposing 64-bit
// reads.  ds_read_b64_tr_b16 hands lane i of a 16-lane group element i%4 of
// the 64 bits read by lane 4j + i/4, j = 0..3; so source lane s of group q
// reads the 4 columns 16*(q%2) + 4*(s%4) .. +3 of K-row 8*(q/2) + s/4 (+4 for
// the second read) and every lane receives its own column's 4 K values.
// addr: this lane's byte address for (32-block, K-slice 0, first read);
// slice ks adds 16*ks rows, the second read 4 rows.
__device__ __forceinline__ u32x4 frag_tr(const uint8_t* stage, uint32_t addr, int ks) {
  const uint8_t* p = stage + addr + ks * 16 * 512;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)((__attribute__((address_space(3))) uint8_t*)(__attribute__((address_space(3))) void*)p));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)((__attribute__((address_space(3))) uint8_t*)(__attribute__((address_space(3))) void*)(p + 4 * 512)));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// Per-lane byte address of the first transposing read of 32-block b (0..3) of
// a wave's 128 columns starting at column c0 (a multiple of 128): K-row
// k = 8*(q/2) + s/4 and column m = c0 + 32b + 16*(q%2) + 4*(s%4), chunk
// m/8 swizzled by 4*(k%4) = 4*(s/4).
__device__ __forceinline__ uint32_t tr_addr(int lane, int c0, int b) {
  const int q = lane >> 4, s = lane & 15;
  const int k = 8 * (q >> 1) + (s >> 2);
  const int chunk = (c0 >> 3) + 4 * (b ^ (s >> 2)) + 2 * (q & 1) + ((s & 3) >> 1);
  return static_cast<uint32_t>(k * 512 + chunk * 16 + 8 * (s & 1));
}

// Block-scaled MFMA with the scale byte chosen by `sel` (a constant after
// unrolling; the instruction takes it as an immediate).
template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma_scaled(i32x8 a, i32x8 b, f32x16 c, int sa, int sb, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, sa, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 1, sa, 1, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 2, sa, 2, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 3, sa, 3, sb);
  }
}

// Scheduling hint for one K-slice: 16 MFMA, each followed by its share of
// the R fragment reads of the next slice and of the V global loads issued in
// this slice.
template <int I, int R, int V>
__device__ __forceinline__ void sched_slice() {
  if constexpr (I < 16) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int n = (I + 1) * R / 16 - I * R / 16;
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, 0);
    constexpr int v = (I + 1) * V / 16 - I * V / 16;
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
    sched_slice<I + 1, R, V>();
  }
}

// The second half of a slice that is split by the block barrier: 8 MFMA with
// the next step's R first fragment reads spread among them.
template <int I, int R>
__device__ __forceinline__ void sched_half() {
  if constexpr (I < 8) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int n = (I + 1) * R / 8 - I * R / 8;
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, 0);
    sched_half<I + 1, R>();
  }
}

// Epilogue through LDS: a wave's MB x NB accumulator blocks of 32x32 (lane l
// holds column l%32 and rows 8*(r/4) + 4*(l/32) + r%4 in element r) leave as
// whole rows of 16-byte non-temporal stores instead of 2- or 4-byte ones.
// One 32-row band at a time goes through this wave's LDS region `buf` (32
// rows; the pitch is the row's bytes + 32, which puts the two half-waves'
// writes on disjoint banks); the block barriers around each band keep every
// wave's region clear of the main loop's fragment reads and of the previous
// band.  C and its rows must be 16-byte aligned.  (The output address is a
// running per-lane pointer: computing it from the tile origin in every pass
// left the compiler short of scalar registers for the direct-to-LDS loads.)
template <int CT, int MB, int NB>
__device__ __forceinline__ void store_tile_lds(const f32x16 (&acc)[MB][NB], float alpha, void* C, int64_t ldc,
                                               int64_t row0, int64_t col0, uint8_t* buf) {
  constexpr int kES = CT == AMP_F32 ? 4 : 2;
  constexpr int kRow = NB * 32 * kES;
  constexpr int kPitch = kRow + 32;
  constexpr int kLPR = kRow / 16;   // lanes per row on the way out
  constexpr int kRPP = 64 / kLPR;   // rows per pass
  const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
  const int64_t ld_b = ldc * kES;
  uint8_t* out = static_cast<uint8_t*>(C) + row0 * ld_b + col0 * kES + (lane / kLPR) * ld_b + (lane % kLPR) * 16;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        uint8_t* p = buf + (8 * (r >> 2) + 4 * h + (r & 3)) * kPitch + (nb * 32 + l32) * kES;
        const float x = acc[mb][nb][r] * alpha;
        if constexpr (CT == AMP_F32) *reinterpret_cast<float*>(p) = x;
        else if constexpr (CT == AMP_BF16) *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(f32_to_bf16(x));
        else *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(f32_to_f16(x));
      }
    __syncthreads();
#pragma unroll
    for (int ps = 0; ps < 32 / kRPP; ++ps) {
      const int row = ps * kRPP + lane / kLPR, seg = lane % kLPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(buf + row * kPitch + seg * 16);
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + (mb * 32 + ps * kRPP) * ld_b));
    }
  }
}

// LDS bytes of one wave's band in store_tile_lds
template <int CT, int NB>
constexpr int store_band_bytes() { return 32 * (NB * 32 * (CT == AMP_F32 ? 4 : 2) + 32); }

// Every tile full; 16-bit operands may be K- or M/N-contiguous (FP8 ones are
// K-contiguous).  Per K-step: the loads of the
// next step go straight to the idle LDS stage; the fragments of slice s+1 are
// read while slice s runs on the matrix cores; the block-wide barrier sits in
// the last slice, after its fragments are in registers, so the last slice's
// MFMAs overlap the first fragment reads of the next step.
template <int AT, int BT, bool A_KC, bool B_KC, int PATH, int CT>
__global__ __launch_bounds__(kThreads, 1) void gemm_mfma_d2l(GemmArgs g) {
  static_assert((A_KC && B_KC) || PATH == kP16, "M/N-contiguous operands are 16-bit");
  // the two stages are separate objects, so that the compiler can tell the
  // loads into one from the fragment reads of the other
  __shared__ __align__(16) uint8_t smem0[2][kOperandBytes];
  __shared__ __align__(16) uint8_t smem1[2][kOperandBytes];
  constexpr bool kF8 = PATH == kPF8Native || PATH == kPF8Exact || PATH == kPMX8 || PATH == kPMX8E;
  constexpr bool kMX = PATH == kPMX8 || PATH == kPMX4 || PATH == kPMX8E;
  constexpr bool kFP4 = PATH == kPMX4 || PATH == kPFP4D;
  constexpr int BK = kFP4 ? 256 : (kF8 ? 128 : 64);               // K elements per step
  constexpr int EB = kF8 || kFP4 ? 1 : 2;                         // row stride unit (bytes for FP4)
  // fragment reads per step: K-slices of 16 (16-bit), 64 (FP8 native, MX),
  // or pairs of 16-slices (FP8 widened to BF16 in registers)
  constexpr int NS = PATH == kPF8Native || PATH == kPMX8 ? 2 : 4;
  const int64_t nbm = g.M / kBM, nbn = g.N / kBN;
  const int64_t total = nbm * nbn;
  int64_t tile = blockIdx.x;
  if (total % 8 == 0) tile = (tile % 8) * (total / 8) + tile / 8;
  constexpr int64_t kGroup = 8;
  const int64_t group = tile / (kGroup * nbn);
  const int64_t first_m = group * kGroup;
  const int64_t gsz = nbm - first_m < kGroup ? nbm - first_m : kGroup;
  const int64_t in_group = tile % (kGroup * nbn);
  const int64_t m0 = (first_m + in_group % gsz) * kBM, n0 = (in_group / gsz) * kBN;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const int64_t nk = g.K / BK;
  const uint32_t lda_b = static_cast<uint32_t>(g.lda * EB), ldb_b = static_cast<uint32_t>(g.ldb * EB);
  const uint8_t* gA = static_cast<const uint8_t*>(g.A);
  const uint8_t* gB = static_cast<const uint8_t*>(g.B);
  // K-contiguous: the resource covers the tile's 256 rows for every step
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(gA + m0 * g.lda * EB), 0, static_cast<int>(kBM * lda_b), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(gB + n0 * g.ldb * EB), 0, static_cast<int>(kBN * ldb_b), 0x00020000);
  // past the end a step reloads the last one into the idle stage (never
  // read); operand 0 (A) and 1 (B) are fetched in different K-slices
  auto load_part = [&](int64_t kt, int which, uint8_t* dst) {
    const int64_t kc = kt < nk ? kt : nk - 1;
    const uint32_t koff = static_cast<uint32_t>(kc * kRowBytes);
    if (which == 0) {
      if constexpr (A_KC) {
        d2l_stage<!B_KC>(ra, lda_b, koff, dst);
      } else {
        // M-contiguous: the step's 64 K-rows, columns m0 .. m0+255
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(gA + (kc * BK * g.lda + m0) * EB), 0, static_cast<int>(BK * lda_b), 0x00020000);
        d2l_stage_mn(r, lda_b, dst);
      }
    } else {
      if constexpr (B_KC) {
        d2l_stage<!A_KC>(rb, ldb_b, koff, dst + kOperandBytes);
      } else {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(gB + (kc * BK * g.ldb + n0) * EB), 0, static_cast<int>(BK * ldb_b), 0x00020000);
        d2l_stage_mn(r, ldb_b, dst + kOperandBytes);
      }
    }
  };
  // Fragment rows wm*128 + mb*32 + l%32 (A) and wn*128 + nb*32 + l%32 (B).
  // Their swizzle term is g ^ 4*(mb & 1) with g = (l%8) ^ (l%32 / 8), so the
  // LDS address is base + 32*mb rows + ((y ^ c) << 4) with a per-lane y and
  // a compile-time c.
  const int l32 = lane & 31, h = lane >> 5;
  const uint32_t gsw = static_cast<uint32_t>((l32 & 7) ^ (l32 >> 3));
  const uint32_t abase = static_cast<uint32_t>(wm * 128 + l32) * kRowBytes;
  const uint32_t bbase = static_cast<uint32_t>(wn * 128 + l32) * kRowBytes;
  // 8-register operands for the f8f6f4 instruction; an E2M1 operand uses the
  // low 4 registers only (the high half is left undefined)
  using Frag = typename std::conditional<PATH == kPF8Native || PATH == kPMX8 || PATH == kPMX4,
                                         i32x8, u32x4>::type;
  // MX FP8 widened to BF16: this lane's UE8M0 block scales of the step for its
  // 4 rows of A and B (row wm*128 + mb*32 + l%32): 4 bytes, one per 32-K block
  uint32_t scA[4], scB[4], nscA[4], nscB[4];
  auto load_scales = [&](int64_t kt, uint32_t (&a)[4], uint32_t (&b)[4]) {
    if constexpr (PATH == kPMX8E) {
      const int64_t kc = kt < nk ? kt : nk - 1;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        a[mb] = *reinterpret_cast<const uint32_t*>(g.sA + (m0 + wm * 128 + mb * 32 + (lane & 31)) * g.ldsA + kc * 4);
        b[mb] = *reinterpret_cast<const uint32_t*>(g.sB + (n0 + wn * 128 + mb * 32 + (lane & 31)) * g.ldsB + kc * 4);
      }
    }
  };
  // MXFP4 and MX FP8 on the block-scaled instruction: the scales of steps 2p
  // and 2p+1 come with one load per row and lane (8 bytes for E2M1, whose
  // 256-K step spans 8 blocks; 4 for FP8), lane half h reading step 2p + h
  // (with both halves reading the same step, every step cost one load per row
  // and operand, each touching a different cache line).  A lane needs bytes
  // 2ks + h of a step's scales (ks = 0..3 for E2M1, 0..1 for FP8): the lane
  // packs its half's bytes of the step it read into one dword, the other
  // half's into another, and one swap across the lane halves hands each lane
  // its bytes of the other step.  Byte ks of a packed dword is the scale of
  // K-block 2ks + h.
  constexpr bool kPair = PATH == kPMX4 || PATH == kPMX8;
  uint32_t p4A[4][2], p4B[4][2], r4A[4][2], r4B[4][2];  // packed [mb][step & 1]; raw
  auto load_pair = [&](int64_t p) {
    if constexpr (kPair) {
      constexpr int kSB = PATH == kPMX4 ? 8 : 4;           // scale bytes per row and step
      int64_t kc = 2 * p + h;
      kc = kc < nk ? kc : nk - 1;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const uint8_t* pa = g.sA + (m0 + wm * 128 + mb * 32 + (lane & 31)) * g.ldsA + kc * kSB;
        const uint8_t* pb = g.sB + (n0 + wn * 128 + mb * 32 + (lane & 31)) * g.ldsB + kc * kSB;
        if constexpr (PATH == kPMX4) {
          const u32x2 va = *reinterpret_cast<const u32x2*>(pa);
          const u32x2 vb = *reinterpret_cast<const u32x2*>(pb);
          r4A[mb][0] = va[0]; r4A[mb][1] = va[1];
          r4B[mb][0] = vb[0]; r4B[mb][1] = vb[1];
        } else {
          r4A[mb][0] = *reinterpret_cast<const uint32_t*>(pa); r4A[mb][1] = 0u;
          r4B[mb][0] = *reinterpret_cast<const uint32_t*>(pb); r4B[mb][1] = 0u;
        }
      }
    }
  };
  auto unpack_pair = [&]() {
    if constexpr (kPair) {
      // even bytes (lane half 0's) and odd bytes (half 1's) of the 8 (E2M1) or
      // of the 4 (FP8; selector 0x0c gives a zero byte)
      constexpr uint32_t kEven = PATH == kPMX4 ? 0x06040200u : 0x0c0c0200u;
      constexpr uint32_t kOdd = PATH == kPMX4 ? 0x07050301u : 0x0c0c0301u;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const auto sa = __builtin_amdgcn_permlane32_swap(__builtin_amdgcn_perm(r4A[mb][1], r4A[mb][0], kEven),
                                                         __builtin_amdgcn_perm(r4A[mb][1], r4A[mb][0], kOdd),
                                                         false, false);
        const auto sb = __builtin_amdgcn_permlane32_swap(__builtin_amdgcn_perm(r4B[mb][1], r4B[mb][0], kEven),
                                                         __builtin_amdgcn_perm(r4B[mb][1], r4B[mb][0], kOdd),
                                                         false, false);
        p4A[mb][0] = sa[0]; p4A[mb][1] = sa[1];
        p4B[mb][0] = sb[0]; p4B[mb][1] = sb[1];
      }
    }
  };
  // NVFP4: this lane's 16 E4M3 block scales of the step (one per 16 K) for
  // its rows of A and B (16x16 blocks: row / 16)
  u32x4 nvA[4], nvB[4], nnvA[4], nnvB[4];
  auto load_nv = [&](int64_t kt, u32x4 (&a)[4], u32x4 (&b)[4]) {
    if constexpr (PATH == kPFP4D) {
      const int64_t kc = kt < nk ? kt : nk - 1;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int64_t ra_ = m0 + wm * 128 + mb * 32 + (lane & 31);
        const int64_t rb_ = n0 + wn * 128 + mb * 32 + (lane & 31);
        a[mb] = *reinterpret_cast<const u32x4*>(g.sA + (g.s2dA ? ra_ / 16 : ra_) * g.ldsA + kc * 16);
        b[mb] = *reinterpret_cast<const u32x4*>(g.sB + (g.s2dB ? rb_ / 16 : rb_) * g.ldsB + kc * 16);
      }
    }
  };
  Frag fa[2][4], fb[2][4];
  uint32_t tra[4], trb[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    tra[b] = tr_addr(lane, wm * 128, b);
    trb[b] = tr_addr(lane, wn * 128, b);
  }
  auto frag = [&](const uint8_t* st, int ks, Frag (&a)[4], Frag (&b)[4]) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if constexpr (PATH == kPF8Native || PATH == kPMX8) {
        // 32 bytes of K per lane.  Native FP8: logical chunks 4ks + 2h and
        // 4ks + 2h + 1 (any K order shared by A and B will do).  MX: the
        // instruction's K block 0 is made of bytes 0-15 of both lane halves
        // and block 1 of bytes 16-31, so lane half h takes chunks 4ks + h
        // (16 elements of MX block 2ks) and 4ks + 2 + h (of block 2ks + 1)
        constexpr bool kMXO = PATH == kPMX8;
        const uint32_t y = (static_cast<uint32_t>(kMXO ? h : 2 * h) ^ gsw) & 7u;
        const uint32_t c0 = static_cast<uint32_t>(4 * ks) ^ static_cast<uint32_t>(4 * (mb & 1));
        const uint32_t c1 = c0 + (kMXO ? 2u : 1u);
        const uint8_t* pa = st + abase + mb * 32 * kRowBytes;
        const uint8_t* pb = st + kOperandBytes + bbase + mb * 32 * kRowBytes;
        const u32x4 al = *reinterpret_cast<const u32x4*>(pa + ((y ^ c0) << 4));
        const u32x4 ah = *reinterpret_cast<const u32x4*>(pa + ((y ^ c1) << 4));
        const u32x4 bl = *reinterpret_cast<const u32x4*>(pb + ((y ^ c0) << 4));
        const u32x4 bh = *reinterpret_cast<const u32x4*>(pb + ((y ^ c1) << 4));
        a[mb] = i32x8{(int)al[0], (int)al[1], (int)al[2], (int)al[3], (int)ah[0], (int)ah[1], (int)ah[2], (int)ah[3]};
        b[mb] = i32x8{(int)bl[0], (int)bl[1], (int)bl[2], (int)bl[3], (int)bh[0], (int)bh[1], (int)bh[2], (int)bh[3]};
      } else if constexpr (PATH == kPMX4) {
        // 16 bytes = 32 E2M1 of K per lane: logical chunk 2ks + h (MX block 2ks + h)
        const uint32_t y = (static_cast<uint32_t>(h) ^ gsw) & 7u;
        const uint32_t c = static_cast<uint32_t>(2 * ks) ^ static_cast<uint32_t>(4 * (mb & 1));
        const i32x4 av = *reinterpret_cast<const i32x4*>(st + abase + mb * 32 * kRowBytes + ((y ^ c) << 4));
        const i32x4 bv = *reinterpret_cast<const i32x4*>(st + kOperandBytes + bbase + mb * 32 * kRowBytes +
                                                         ((y ^ c) << 4));
        a[mb] = __builtin_shufflevector(av, av, 0, 1, 2, 3, -1, -1, -1, -1);
        b[mb] = __builtin_shufflevector(bv, bv, 0, 1, 2, 3, -1, -1, -1, -1);
      } else {
        // 16 bytes of K per lane: logical chunk 2ks + h
        const uint32_t y = (static_cast<uint32_t>(h) ^ gsw) & 7u;
        const uint32_t c = static_cast<uint32_t>(2 * ks) ^ static_cast<uint32_t>(4 * (mb & 1));
        if constexpr (A_KC)
          a[mb] = *reinterpret_cast<const u32x4*>(st + abase + mb * 32 * kRowBytes + ((y ^ c) << 4));
        else
          a[mb] = frag_tr(st, tra[mb], ks);
        if constexpr (B_KC)
          b[mb] = *reinterpret_cast<const u32x4*>(st + kOperandBytes + bbase + mb * 32 * kRowBytes +
                                                  ((y ^ c) << 4));
        else
          b[mb] = frag_tr(st + kOperandBytes, trb[mb], ks);
      }
    }
  };
  load_part(0, 0, smem0[0]);
  load_part(0, 1, smem0[0]);
  if constexpr (kPair) load_pair(0); else load_scales(0, scA, scB);
  load_nv(0, nvA, nvB);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  unpack_pair();
  frag(smem0[0], 0, fa[0], fb[0]);
  // par = kt & 1 (a constant at every call site of the MXFP4 path)
  auto step = [&](int64_t kt, const uint8_t* st, uint8_t* nst, int par) __attribute__((always_inline)) {
    if constexpr (kPair) {
      if (par == 0) load_pair(kt / 2 + 1);
    } else {
      load_scales(kt + 1, nscA, nscB);
    }
    load_nv(kt + 1, nnvA, nnvB);
    // The next step's scales are consumed only after the closing barrier;
    // left to itself the scheduler sinks their loads to just before that
    // barrier's vmcnt(0), exposing their latency once per step.
    if constexpr (kMX || PATH == kPFP4D) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < NS; ++ks) {
      const int cur = ks & 1;
      // K-contiguous operands: A's loads in slice 0 and B's in slice 1, spread
      // among the MFMAs; with transposed operands both at the start of the
      // step, and with only two slices per step both in slice 0 (B's loads
      // in the last slice would meet the barrier's wait at once)
      constexpr bool kSplit = A_KC && B_KC && NS > 2;
      if (kSplit && ks < 2) load_part(kt + 1, ks, nst);
      if (!kSplit && ks == 0) {
        load_part(kt + 1, 0, nst);
        load_part(kt + 1, 1, nst);
      }
      // With two slices per step (FP8 elements, 64 K per MFMA) the barrier
      // moves to the middle of the last slice: the loads of the first slice
      // get half a slice more to land, and the next step's first fragment
      // reads still overlap 8 MFMAs.  (Measured: +4-8 % there; with four
      // slices the end-of-slice barrier is as fast or faster.)
      constexpr bool kMid = NS == 2;
      auto next_step = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
        frag(nst, 0, fa[cur ^ 1], fb[cur ^ 1]);
      };
      if (ks + 1 < NS) {
        frag(st, ks + 1, fa[cur ^ 1], fb[cur ^ 1]);
      } else if (!kMid) {
        next_step();
      }
      if constexpr (PATH == kPFP4D) {
        // 16 bytes = 32 E2M1 of K per lane (logical chunk c = 2ks + h, NVFP4
        // blocks 2c and 2c+1 of the step); dword e holds the 8 K values this
        // lane gives MFMA e, scaled by block 2c + e/2
        f16x2_t sa2[4], sb2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sa2[i] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(nvA[i][ks] >> (16 * h), 1.0f, false));
          sb2[i] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(nvB[i][ks] >> (16 * h), 1.0f, false));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u32x4 da[4], db[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f16x2_t a2 = e < 2 ? f16x2_t{sa2[i][0], sa2[i][0]} : f16x2_t{sa2[i][1], sa2[i][1]};
            const f16x2_t b2 = e < 2 ? f16x2_t{sb2[i][0], sb2[i][0]} : f16x2_t{sb2[i][1], sb2[i][1]};
            da[i] = fp4x8_to_f16(fa[cur][i][e], a2);
            db[i] = fp4x8_to_f16(fb[cur][i][e], b2);
          }
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, da[mb]),
                                                                   __builtin_bit_cast(f16x8_t, db[nb]),
                                                                   acc[mb][nb], 0, 0, 0);
        }
      } else if constexpr (PATH == kPF8Exact || PATH == kPMX8E) {
        // 16 FP8 bytes per lane = K 32p + 16h + 8e + j for e = 0, 1: two BF16
        // fragments (the same K order for A and B; products are exact).  MX:
        // slice ks is MX block ks of the step for both lane halves, and the
        // conversion multiplies by that block's power-of-two scale
        u32x4 da[2][4], db[2][4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          float sa = 1.0f, sb = 1.0f;
          if constexpr (PATH == kPMX8E) {
            sa = e8m0_scale((scA[mb] >> (8 * ks)) & 0xffu);
            sb = e8m0_scale((scB[mb] >> (8 * ks)) & 0xffu);
          }
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            da[e][mb] = u32x4{fp8x2_to_bf16x2<AT, false>(fa[cur][mb][2 * e], sa), fp8x2_to_bf16x2<AT, true>(fa[cur][mb][2 * e], sa),
                              fp8x2_to_bf16x2<AT, false>(fa[cur][mb][2 * e + 1], sa), fp8x2_to_bf16x2<AT, true>(fa[cur][mb][2 * e + 1], sa)};
            db[e][mb] = u32x4{fp8x2_to_bf16x2<BT, false>(fb[cur][mb][2 * e], sb), fp8x2_to_bf16x2<BT, true>(fb[cur][mb][2 * e], sb),
                              fp8x2_to_bf16x2<BT, false>(fb[cur][mb][2 * e + 1], sb), fp8x2_to_bf16x2<BT, true>(fb[cur][mb][2 * e + 1], sb)};
          }
        }
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, da[e][mb]),
                                                                    __builtin_bit_cast(bf16x8_t, db[e][nb]),
                                                                    acc[mb][nb], 0, 0, 0);
      } else {
      auto rows = [&](int mb0, int mb1) __attribute__((always_inline)) {
#pragma unroll
      for (int mb = mb0; mb < mb1; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          if constexpr (PATH == kPF8Native) {
            constexpr int fa_ = AT == AMP_E4M3 ? 0 : 1;
            constexpr int fb_ = BT == AMP_E4M3 ? 0 : 1;
            acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[cur][mb], fb[cur][nb], acc[mb][nb],
                                                                          fa_, fb_, 0, 127, 0, 127);
          } else if constexpr (PATH == kPMX8) {
            // lane l covers K block 2ks + l/32 of the step: its scale byte is
            // byte ks of the packed dword
            constexpr int fa_ = AT == AMP_E4M3 ? 0 : 1;
            constexpr int fb_ = BT == AMP_E4M3 ? 0 : 1;
            const int sa = static_cast<int>(p4A[mb][par]);
            const int sb = static_cast<int>(p4B[nb][par]);
            acc[mb][nb] = mfma_scaled<fa_, fb_>(fa[cur][mb], fb[cur][nb], acc[mb][nb], sa, sb, ks);
          } else if constexpr (PATH == kPMX4) {
            // E2M1 (format 4): 16 bytes = 32 K per lane in the low 4 dwords
            const i32x8 av = fa[cur][mb], bv = fb[cur][nb];
            const int sa = static_cast<int>(p4A[mb][par]);
            const int sb = static_cast<int>(p4B[nb][par]);
            acc[mb][nb] = mfma_scaled<4, 4>(av, bv, acc[mb][nb], sa, sb, ks);
          } else if constexpr (AT == AMP_F16) {
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, fa[cur][mb]),
                                                                 __builtin_bit_cast(f16x8_t, fb[cur][nb]),
                                                                 acc[mb][nb], 0, 0, 0);
          } else {
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa[cur][mb]),
                                                                  __builtin_bit_cast(bf16x8_t, fb[cur][nb]),
                                                                  acc[mb][nb], 0, 0, 0);
          }
        }
      };
      if (!kMid || ks + 1 < NS) {
        rows(0, 4);
      } else {
        rows(0, 2);
        __builtin_amdgcn_sched_barrier(0);
        next_step();
        rows(2, 4);
      }
      }
      // 16 MFMA per slice with the next slice's fragment reads spread evenly
      // (8 reads; 16 for FP8; two per transposed fragment)
      constexpr int kReads = PATH == kPF8Native || PATH == kPMX8 ? 16 : (A_KC ? 4 : 8) + (B_KC ? 4 : 8);
      if constexpr (PATH != kPF8Exact && PATH != kPFP4D && PATH != kPMX8E) {
        if (kSplit && ks < 2) sched_slice<0, kReads, 8>();
        else if (!kSplit && A_KC && B_KC && ks == 0) sched_slice<0, kReads, 16>();
        else if (kMid && ks + 1 == NS) sched_half<0, kReads>();
        else sched_slice<0, kReads, 0>();
      }
    }
    // and the register copies stay after the barrier (whose vmcnt(0) they
    // then need not add to)
    if constexpr (kMX || PATH == kPFP4D) __builtin_amdgcn_sched_barrier(0);
    if constexpr (kPair) {
      if (par == 1) unpack_pair();
    } else if constexpr (kMX) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        scA[mb] = nscA[mb];
        scB[mb] = nscB[mb];
      }
    }
    if constexpr (PATH == kPFP4D) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        nvA[mb] = nnvA[mb];
        nvB[mb] = nnvB[mb];
      }
    }
  };
  if constexpr (PATH == kPF8Exact || PATH == kPFP4D || PATH == kPMX8E) {
    // long step bodies without scheduling hints: one step per iteration,
    // stages chosen at run time (measured faster for the first two)
    for (int64_t kt = 0; kt < nk; ++kt)
      step(kt, (kt & 1) ? smem1[0] : smem0[0], (kt & 1) ? smem0[0] : smem1[0], static_cast<int>(kt & 1));
  } else {
    // two steps per iteration, each naming its stages statically
    int64_t kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      step(kt, smem0[0], smem1[0], 0);
      step(kt + 1, smem1[0], smem0[0], 1);
    }
    if (kt < nk) step(kt, smem0[0], smem1[0], 0);
  }
  const float alpha = (g.alphaA ? *g.alphaA : 1.0f) * (g.alphaB ? *g.alphaB : 1.0f);
  constexpr int kES = CT == AMP_F32 ? 4 : 2;
  if ((reinterpret_cast<uintptr_t>(g.C) & 15) == 0 && (g.ldc * kES) % 16 == 0) {
    // waves 0-1 stage their bands in smem0, waves 2-3 in smem1
    static_assert(2 * store_band_bytes<CT, 4>() <= 2 * kOperandBytes, "band staging exceeds a stage");
    store_tile_lds<CT, 4, 4>(acc, alpha, g.C, g.ldc, m0 + wm * 128, n0 + wn * 128,
                             (wave < 2 ? smem0[0] : smem1[0]) + (wave & 1) * store_band_bytes<CT, 4>());
  } else {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int64_t col = n0 + wn * 128 + nb * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm * 128 + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          store_c<CT>(g.C, row * g.ldc + col, acc[mb][nb][r] * alpha);
        }
      }
  }
}

// ---------------------------------------------------------------- generic
// Any shape, stride and layout (small or odd GEMMs): one output per thread,
// operands widened exactly to FP32, products exact, FP32 fused accumulation.
template <int ET>
__device__ __forceinline__ float load_elem(const void* X, int64_t idx) {
  if constexpr (ET == AMP_BF16) return bf16_to_f32(static_cast<const uint16_t*>(X)[idx]);
  else if constexpr (ET == AMP_F16) return f16_to_f32(static_cast<const uint16_t*>(X)[idx]);
  else if constexpr (ET == AMP_E4M3) return e4m3_to_f32(static_cast<const uint8_t*>(X)[idx]);
  else return e5m2_to_f32(static_cast<const uint8_t*>(X)[idx]);
}

template <int ET>
__device__ __forceinline__ float operand(const void* X, int64_t ld, bool kc, int64_t r, int64_t k,
                                         const uint8_t* sc, int64_t lds_, int s2d, int mx) {
  float v;
  if constexpr (ET == AMP_E2M1X2) {
    const uint8_t byte = static_cast<const uint8_t*>(X)[r * ld + k / 2];
    v = e2m1_to_f32((k & 1) ? (byte >> 4) : (byte & 0xf));
  } else {
    v = load_elem<ET>(X, kc ? r * ld + k : k * ld + r);
  }
  if (mx) {
    // UE8M0 per 32 along K: 2^(code - 127), 0xFF = NaN
    const uint32_t c = sc[r * lds_ + k / 32];
    const float S = c == 0xffu ? __builtin_nanf("") : __builtin_ldexpf(1.0f, static_cast<int>(c) - 127);
    return v * S;
  }
  if constexpr (ET == AMP_E2M1X2) return v * e4m3_to_f32(sc[(s2d ? r / 16 : r) * lds_ + k / 16]);
  return v;
}

template <int AT, int BT, int CT>
__global__ __launch_bounds__(256) void gemm_generic(GemmArgs g, int a_kc, int b_kc) {
  const int64_t col = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x & 15);
  const int64_t row = static_cast<int64_t>(blockIdx.y) * 16 + (threadIdx.x >> 4);
  if (row >= g.M || col >= g.N) return;
  float acc = 0.0f;
  for (int64_t k = 0; k < g.K; ++k) {
    const float a = operand<AT>(g.A, g.lda, a_kc, row, k, g.sA, g.ldsA, g.s2dA, g.mx);
    const float b = operand<BT>(g.B, g.ldb, b_kc, col, k, g.sB, g.ldsB, g.s2dB, g.mx);
    acc = __builtin_fmaf(a, b, acc);
  }
  const float alpha = (g.alphaA ? *g.alphaA : 1.0f) * (g.alphaB ? *g.alphaB : 1.0f);
  store_c<CT>(g.C, row * g.ldc + col, acc * alpha);
}

// An empty sum (K == 0): C = +0 everywhere; neither operand nor scale is read.
template <int CT>
__global__ __launch_bounds__(256) void gemm_zero(GemmArgs g) {
  const int64_t col = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x & 15);
  const int64_t row = static_cast<int64_t>(blockIdx.y) * 16 + (threadIdx.x >> 4);
  if (row >= g.M || col >= g.N) return;
  store_c<CT>(g.C, row * g.ldc + col, 0.0f);
}


// ------------------------------------------- fine-grained FP8 (blockwise)
// Page itwiki, section "FP8 혼합 정밀도": DeepSeek-V3's operands carry one
// FP32 scale per 1x128 tile (activations, gradients) or 128x128 block
// (weights); page hwlabs, section "GEMM 누적 정밀도 문제": each tile's
// partial sum is promoted to an FP32 accumulator.  Here every 128-K block's
// partial sum P (exact FP8 products widened to BF16, FP32 matrix-core sums)
// is added as C += P * fl32(sa * sb).
//
// Shape: one 512-thread block (8 waves, 4x2) per 256x128 output tile, each
// wave 64x64 = 2x2 MFMA 32x32 blocks, with 16 FP32 accumulators and 16
// partial-sum registers per block (two waves per SIMD).  The K-step is the
// 128-element scale block; A, B and the step's 256 A-row scales travel to
// LDS by direct-to-LDS loads.  A's scales are per row, B's per row or per
// 128-row block.

struct BwArgs {
  const uint8_t* A;
  const uint8_t* B;
  void* C;
  int64_t M, N, K, lda, ldb, ldc;
  const float* sA;
  const float* sB;
  int64_t ldsA, ldsB;
  int a_block, b_block;
};

constexpr int kBwBM = 256, kBwBN = 128, kBwThreads = 512;

// A stage of ROWS 128-byte rows filled by NW waves (ROWS / NW rows each, 8
// rows per 1 KB load), in the XOR-swizzled layout of swz().
template <int ROWS, int NW>
__device__ __forceinline__ void d2l_rows(__amdgpu_buffer_rsrc_t rsrc, uint32_t ld, uint32_t koff,
                                         uint8_t* stage) {
  constexpr int RPW = ROWS / NW;
  static_assert(RPW % 8 == 0, "whole 8-row loads per wave");
  const int lane = threadIdx.x & 63, w = wave_id();
  const uint32_t vrow = static_cast<uint32_t>(w * RPW + lane / 8) * ld;
  const uint32_t x = static_cast<uint32_t>((lane & 7) ^ (lane >> 3));
#pragma unroll
  for (int i = 0; i < RPW / 8; ++i) {
    const uint32_t chunk = (x ^ static_cast<uint32_t>(w * (RPW / 8) + i)) & 7u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(stage + (w * RPW + i * 8) * kRowBytes),
                                             16, vrow + (chunk << 4),
                                             koff + static_cast<uint32_t>(8 * i) * ld, 0, 0);
  }
}

template <int AT, int BT, bool B_BLOCK, int CT>
__global__ __launch_bounds__(kBwThreads, 1) void gemm_bw_d2l(BwArgs g) {
  constexpr int kOffB = kBwBM * kRowBytes;                  // B rows after A's
  constexpr int kOffS = kOffB + kBwBN * kRowBytes;          // then A's 256 scales
  constexpr int kStage = kOffS + kBwBM * 4;
  // two stage objects, named statically two K-blocks at a time, so that the
  // compiler can tell one stage's loads from the other's fragment reads
  __shared__ __align__(16) uint8_t smem0[kStage];
  __shared__ __align__(16) uint8_t smem1[kStage];
  const int64_t nbm = g.M / kBwBM, nbn = g.N / kBwBN;
  const int64_t total = nbm * nbn;
  int64_t tile = blockIdx.x;
  if (total % 8 == 0) tile = (tile % 8) * (total / 8) + tile / 8;
  constexpr int64_t kGroup = 8;
  const int64_t group = tile / (kGroup * nbn);
  const int64_t first_m = group * kGroup;
  const int64_t gsz = nbm - first_m < kGroup ? nbm - first_m : kGroup;
  const int64_t in_group = tile % (kGroup * nbn);
  const int64_t m0 = (first_m + in_group % gsz) * kBwBM, n0 = (in_group / gsz) * kBwBN;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;
  f32x16 acc[2][2], P[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const f32x16 zero = {};
  const int64_t nk = g.K / 128;
  const uint32_t lda = static_cast<uint32_t>(g.lda), ldb = static_cast<uint32_t>(g.ldb);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(g.A + m0 * g.lda), 0, static_cast<int>(kBwBM * lda), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(g.B + n0 * g.ldb), 0, static_cast<int>(kBwBN * ldb), 0x00020000);
  // A's scales of K-block kb: 256 floats at sA[kb * ldsA + m0 ..]
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(g.sA + m0), 0, static_cast<int>(((nk - 1) * g.ldsA + kBwBM) * 4), 0x00020000);
  // past the end a step reloads the last one into the idle stage (never read)
  auto load_part = [&](int64_t kt, int which, uint8_t* st) {
    const int64_t kc = kt < nk ? kt : nk - 1;
    if (which == 0) {
      d2l_rows<kBwBM, 8>(ra, lda, static_cast<uint32_t>(kc * 128), st);
      if (wave == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(st + kOffS), 16,
                                                 static_cast<uint32_t>(lane * 16),
                                                 static_cast<uint32_t>(kc * g.ldsA * 4), 0, 0);
    } else {
      d2l_rows<kBwBN, 8>(rb, ldb, static_cast<uint32_t>(kc * 128), st + kOffB);
    }
  };
  // B's scales for this lane's columns n0 + wn*64 + nb*32 + l%32 (one value
  // per wave in block mode), fetched one step ahead
  float sb[2], nsb[2];
  auto load_sb = [&](int64_t kt, float (&v)[2]) {
    const int64_t kc = kt < nk ? kt : nk - 1;
    if constexpr (B_BLOCK) {
      v[0] = v[1] = g.sB[kc * g.ldsB + (n0 >> 7)];
    } else {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) v[nb] = g.sB[kc * g.ldsB + n0 + wn * 64 + nb * 32 + l32];
    }
  };
  const uint32_t gsw = static_cast<uint32_t>((l32 & 7) ^ (l32 >> 3));
  const uint32_t abase = static_cast<uint32_t>(wm * 64 + l32) * kRowBytes;
  const uint32_t bbase = kOffB + static_cast<uint32_t>(wn * 64 + l32) * kRowBytes;
  u32x4 fa[2][2], fb[2][2];
  // slice ks: 16 FP8 bytes per lane = logical chunk 2ks + h of rows
  // wm*64 + mb*32 + l%32 (A) and wn*64 + nb*32 + l%32 (B)
  auto frag = [&](const uint8_t* st, int ks, u32x4 (&a)[2], u32x4 (&b)[2]) {
    const uint32_t y = (static_cast<uint32_t>(h) ^ gsw) & 7u;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t c = static_cast<uint32_t>(2 * ks) ^ static_cast<uint32_t>(4 * (i & 1));
      a[i] = *reinterpret_cast<const u32x4*>(st + abase + i * 32 * kRowBytes + ((y ^ c) << 4));
      b[i] = *reinterpret_cast<const u32x4*>(st + bbase + i * 32 * kRowBytes + ((y ^ c) << 4));
    }
  };
  load_part(0, 0, smem0);
  load_part(0, 1, smem0);
  load_sb(0, sb);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  frag(smem0, 0, fa[0], fb[0]);
  auto step = [&](int64_t kt, const uint8_t* st, uint8_t* nst) __attribute__((always_inline)) {
    load_sb(kt + 1, nsb);
    f32x4 sav[2][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int cur = ks & 1;
      if (ks < 2) load_part(kt + 1, ks, nst);
      if (ks < 3) {
        frag(st, ks + 1, fa[cur ^ 1], fb[cur ^ 1]);
      } else {
        // this step's A-row scales: rows wm*64 + mb*32 + 8q + 4h + (0..3)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            sav[mb][q4] = *reinterpret_cast<const f32x4*>(st + kOffS + (wm * 64 + mb * 32 + 8 * q4 + 4 * h) * 4);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
        frag(nst, 0, fa[cur ^ 1], fb[cur ^ 1]);
      }
      u32x4 da[2][2], db[2][2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          da[e][i] = u32x4{fp8x2_to_bf16x2<AT, false>(fa[cur][i][2 * e]), fp8x2_to_bf16x2<AT, true>(fa[cur][i][2 * e]),
                           fp8x2_to_bf16x2<AT, false>(fa[cur][i][2 * e + 1]), fp8x2_to_bf16x2<AT, true>(fa[cur][i][2 * e + 1])};
          db[e][i] = u32x4{fp8x2_to_bf16x2<BT, false>(fb[cur][i][2 * e]), fp8x2_to_bf16x2<BT, true>(fb[cur][i][2 * e]),
                           fp8x2_to_bf16x2<BT, false>(fb[cur][i][2 * e + 1]), fp8x2_to_bf16x2<BT, true>(fb[cur][i][2 * e + 1])};
        }
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            P[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, da[e][mb]), __builtin_bit_cast(bf16x8_t, db[e][nb]),
                (ks == 0 && e == 0) ? zero : P[mb][nb], 0, 0, 0);
    }
    // promote the K-block's partial sums: acc += P * fl32(sa * sb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float sc = sav[mb][r >> 2][r & 3] * sb[nb];
          acc[mb][nb][r] = __builtin_fmaf(P[mb][nb][r], sc, acc[mb][nb][r]);
        }
    sb[0] = nsb[0];
    sb[1] = nsb[1];
  };
  int64_t kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, smem0, smem1);
    step(kt + 1, smem1, smem0);
  }
  if (kt < nk) step(kt, smem0, smem1);
  constexpr int kES = CT == AMP_F32 ? 4 : 2;
  if ((reinterpret_cast<uintptr_t>(g.C) & 15) == 0 && (g.ldc * kES) % 16 == 0) {
    // waves 0-3 stage their bands in smem0, waves 4-7 in smem1
    static_assert(4 * store_band_bytes<CT, 2>() <= kStage, "band staging exceeds a stage");
    store_tile_lds<CT, 2, 2>(acc, 1.0f, g.C, g.ldc, m0 + wm * 64, n0 + wn * 64,
                             (wave < 4 ? smem0 : smem1) + (wave & 3) * store_band_bytes<CT, 2>());
  } else {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int64_t col = n0 + wn * 64 + nb * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm * 64 + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          store_c<CT>(g.C, row * g.ldc + col, acc[mb][nb][r]);
        }
      }
  }
}

// Any shape: one output per thread; each K-block's exact products are summed
// in FP32 and promoted with its scales.
template <int AT, int BT, int CT>
__global__ __launch_bounds__(256) void gemm_bw_generic(BwArgs g) {
  const int64_t col = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x & 15);
  const int64_t row = static_cast<int64_t>(blockIdx.y) * 16 + (threadIdx.x >> 4);
  if (row >= g.M || col >= g.N) return;
  float acc = 0.0f;
  for (int64_t k0 = 0; k0 < g.K; k0 += 128) {
    const int64_t k1 = k0 + 128 < g.K ? k0 + 128 : g.K;
    float p = 0.0f;
    for (int64_t k = k0; k < k1; ++k)
      p = __builtin_fmaf(load_elem<AT>(g.A, row * g.lda + k), load_elem<BT>(g.B, col * g.ldb + k), p);
    const int64_t kb = k0 / 128;
    const float sa = g.sA[kb * g.ldsA + (g.a_block ? row / 128 : row)];
    const float sb = g.sB[kb * g.ldsB + (g.b_block ? col / 128 : col)];
    acc = __builtin_fmaf(p, sa * sb, acc);
  }
  store_c<CT>(g.C, row * g.ldc + col, acc);
}

template <int AT, int BT>
hipError_t launch_bw_t(const BwArgs& g, bool fast, int ct, hipStream_t s) {
  if (fast) {
    const dim3 grid(static_cast<unsigned>((g.M / kBwBM) * (g.N / kBwBN)));
#define AMP_BWK(BB)                                                                              \
    switch (ct) {                                                                               \
      case AMP_F32: gemm_bw_d2l<AT, BT, BB, AMP_F32><<<grid, kBwThreads, 0, s>>>(g); break;     \
      case AMP_BF16: gemm_bw_d2l<AT, BT, BB, AMP_BF16><<<grid, kBwThreads, 0, s>>>(g); break;   \
      default: gemm_bw_d2l<AT, BT, BB, AMP_F16><<<grid, kBwThreads, 0, s>>>(g); break;          \
    }
    if (g.b_block) { AMP_BWK(true) } else { AMP_BWK(false) }
#undef AMP_BWK
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>((g.N + 15) / 16), static_cast<unsigned>((g.M + 15) / 16));
  switch (ct) {
    case AMP_F32: gemm_bw_generic<AT, BT, AMP_F32><<<grid, 256, 0, s>>>(g); break;
    case AMP_BF16: gemm_bw_generic<AT, BT, AMP_BF16><<<grid, 256, 0, s>>>(g); break;
    default: gemm_bw_generic<AT, BT, AMP_F16><<<grid, 256, 0, s>>>(g); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- dispatch
template <int AT, int BT, bool A_KC, bool B_KC, int PATH, bool CHECK>
hipError_t launch_mfma_c(const GemmArgs& g, int ct, hipStream_t s) {
  const int64_t tiles = ((g.M + kBM - 1) / kBM) * ((g.N + kBN - 1) / kBN);
  const dim3 grid(static_cast<unsigned>(tiles));
  switch (ct) {
    case AMP_F32: gemm_mfma<AT, BT, A_KC, B_KC, PATH, AMP_F32, CHECK><<<grid, kThreads, 0, s>>>(g); break;
    case AMP_BF16: gemm_mfma<AT, BT, A_KC, B_KC, PATH, AMP_BF16, CHECK><<<grid, kThreads, 0, s>>>(g); break;
    default: gemm_mfma<AT, BT, A_KC, B_KC, PATH, AMP_F16, CHECK><<<grid, kThreads, 0, s>>>(g); break;
  }
  return hipGetLastError();
}

// Interior launches (every tile full, K a multiple of the K-step) use the
// loaders without bounds checks.
template <int AT, int BT, bool A_KC, bool B_KC, int PATH>
hipError_t launch_mfma(const GemmArgs& g, int ct, hipStream_t s) {
  constexpr int64_t BK = PATH == kPF8Native ? 128 : 64;
  if constexpr ((A_KC && B_KC && (PATH == kP16 || PATH == kPF8Native || PATH == kPF8Exact)) ||
                PATH == kP16) {
    const int eb = PATH == kPF8Native || PATH == kPF8Exact ? 1 : 2;
    // buffer offsets are 32-bit: a 256-row (K-contiguous) or 64-K-row (M/N-
    // contiguous) window of either operand must span < 2 GiB; M/N-contiguous
    // rows hold 256-column windows at 16-byte boundaries
    const int64_t wa = g.lda * eb * (A_KC ? kBM : BK), wb = g.ldb * eb * (B_KC ? kBN : BK);
    const bool small = wa < (int64_t(1) << 31) && wb < (int64_t(1) << 31);
    const int64_t bk_d2l = eb == 1 ? 128 : 64;      // 128 bytes of K per row and step
    if (g.M % kBM == 0 && g.N % kBN == 0 && g.K % bk_d2l == 0 && (g.lda * eb) % 16 == 0 &&
        (g.ldb * eb) % 16 == 0 && small) {
      const dim3 grid(static_cast<unsigned>((g.M / kBM) * (g.N / kBN)));
      switch (ct) {
        case AMP_F32: gemm_mfma_d2l<AT, BT, A_KC, B_KC, PATH, AMP_F32><<<grid, kThreads, 0, s>>>(g); break;
        case AMP_BF16: gemm_mfma_d2l<AT, BT, A_KC, B_KC, PATH, AMP_BF16><<<grid, kThreads, 0, s>>>(g); break;
        default: gemm_mfma_d2l<AT, BT, A_KC, B_KC, PATH, AMP_F16><<<grid, kThreads, 0, s>>>(g); break;
      }
      return hipGetLastError();
    }
  }
  if (g.M % kBM == 0 && g.N % kBN == 0 && g.K % BK == 0)
    return launch_mfma_c<AT, BT, A_KC, B_KC, PATH, false>(g, ct, s);
  return launch_mfma_c<AT, BT, A_KC, B_KC, PATH, true>(g, ct, s);
}

template <int AT, int BT>
hipError_t launch_generic(const GemmArgs& g, bool a_kc, bool b_kc, int ct, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((g.N + 15) / 16), static_cast<unsigned>((g.M + 15) / 16));
  switch (ct) {
    case AMP_F32: gemm_generic<AT, BT, AMP_F32><<<grid, 256, 0, s>>>(g, a_kc, b_kc); break;
    case AMP_BF16: gemm_generic<AT, BT, AMP_BF16><<<grid, 256, 0, s>>>(g, a_kc, b_kc); break;
    default: gemm_generic<AT, BT, AMP_F16><<<grid, 256, 0, s>>>(g, a_kc, b_kc); break;
  }
  return hipGetLastError();
}

template <int ET>
hipError_t launch_16(const GemmArgs& g, bool a_kc, bool b_kc, bool fast, int ct, hipStream_t s) {
  if (!fast) return launch_generic<ET, ET>(g, a_kc, b_kc, ct, s);
  if (a_kc && b_kc) return launch_mfma<ET, ET, true, true, kP16>(g, ct, s);
  if (a_kc) return launch_mfma<ET, ET, true, false, kP16>(g, ct, s);
  if (b_kc) return launch_mfma<ET, ET, false, true, kP16>(g, ct, s);
  return launch_mfma<ET, ET, false, false, kP16>(g, ct, s);
}

template <int AT, int BT>
hipError_t launch_f8(const GemmArgs& g, bool fast, bool native, int ct, hipStream_t s) {
  if (!fast) return launch_generic<AT, BT>(g, true, true, ct, s);
  if (native) return launch_mfma<AT, BT, true, true, kPF8Native>(g, ct, s);
  return launch_mfma<AT, BT, true, true, kPF8Exact>(g, ct, s);
}

// MX operands (both K-contiguous): the block-scaled matrix-core path for full
// tiles with aligned rows and scale rows, the generic kernel otherwise.
template <int AT, int BT, int PATH>
hipError_t launch_mx_t(const GemmArgs& g, int ct, hipStream_t s) {
  constexpr int64_t BK = PATH == kPMX4 ? 256 : 128;
  constexpr int64_t kSB = PATH == kPMX4 ? 8 : 4;           // scale bytes per row per step
  const bool fast = g.M % kBM == 0 && g.N % kBN == 0 && g.K % BK == 0 && aligned(g.A, 16) &&
                    aligned(g.B, 16) && g.lda % 16 == 0 && g.ldb % 16 == 0 &&
                    g.lda * kBM < (int64_t(1) << 31) && g.ldb * kBN < (int64_t(1) << 31) &&
                    aligned(g.sA, kSB) && aligned(g.sB, kSB) && g.ldsA % kSB == 0 &&
                    g.ldsB % kSB == 0;
  if (!fast) return launch_generic<AT, BT>(g, true, true, ct, s);
  const dim3 grid(static_cast<unsigned>((g.M / kBM) * (g.N / kBN)));
  switch (ct) {
    case AMP_F32: gemm_mfma_d2l<AT, BT, true, true, PATH, AMP_F32><<<grid, kThreads, 0, s>>>(g); break;
    case AMP_BF16: gemm_mfma_d2l<AT, BT, true, true, PATH, AMP_BF16><<<grid, kThreads, 0, s>>>(g); break;
    default: gemm_mfma_d2l<AT, BT, true, true, PATH, AMP_F16><<<grid, kThreads, 0, s>>>(g); break;
  }
  return hipGetLastError();
}

// FP8 elements: widened exactly to BF16 times the block scale by default;
// `native` takes the block-scaled FP8 instruction (its reduced-precision
// internal sums).  E2M1 elements: the block-scaled instruction (exact enough:
// few product bits).
template <int PATH>
hipError_t launch_mx8(const GemmArgs& g, int at, int bt, int ct, hipStream_t s) {
  if (at == AMP_E4M3 && bt == AMP_E4M3) return launch_mx_t<AMP_E4M3, AMP_E4M3, PATH>(g, ct, s);
  if (at == AMP_E4M3) return launch_mx_t<AMP_E4M3, AMP_E5M2, PATH>(g, ct, s);
  if (bt == AMP_E4M3) return launch_mx_t<AMP_E5M2, AMP_E4M3, PATH>(g, ct, s);
  return launch_mx_t<AMP_E5M2, AMP_E5M2, PATH>(g, ct, s);
}

hipError_t launch_mx(const GemmArgs& g, int at, int bt, int ct, bool native, hipStream_t s) {
  if (at == AMP_E2M1X2) return launch_mx_t<AMP_E2M1X2, AMP_E2M1X2, kPMX4>(g, ct, s);
  if (native) return launch_mx8<kPMX8>(g, at, bt, ct, s);
  return launch_mx8<kPMX8E>(g, at, bt, ct, s);
}

}  // namespace

// fp8_native: use the FP8 matrix-core dot product (reduced internal precision
// of the 64-term partial sums) instead of the exact BF16 route.
hipError_t launch_gemm(int opA, int opB, int64_t M, int64_t N, int64_t K, const void* A,
                       int at, int64_t lda, const float* alphaA, const void* B, int bt,
                       int64_t ldb, const float* alphaB, void* C, int ct, int64_t ldc,
                       const amp_block_scales* bsA, const amp_block_scales* bsB,
                       int flags, hipStream_t s) {
  const bool fp8_native = (flags & AMP_GEMM_FP8_NATIVE) != 0;
  const bool mx = (flags & AMP_GEMM_MX) != 0;
  GemmArgs g{A, B, C, M, N, K, lda, ldb, ldc, alphaA, alphaB,
             bsA ? bsA->scales : nullptr, bsB ? bsB->scales : nullptr,
             bsA ? bsA->ld : 0, bsB ? bsB->ld : 0, bsA ? bsA->block2d : 0,
             bsB ? bsB->block2d : 0, mx ? 1 : 0};
  if (K == 0) {
    // every kernel below assumes at least one K-step
    const dim3 grid(static_cast<unsigned>((N + 15) / 16), static_cast<unsigned>((M + 15) / 16));
    switch (ct) {
      case AMP_F32: gemm_zero<AMP_F32><<<grid, 256, 0, s>>>(g); break;
      case AMP_BF16: gemm_zero<AMP_BF16><<<grid, 256, 0, s>>>(g); break;
      default: gemm_zero<AMP_F16><<<grid, 256, 0, s>>>(g); break;
    }
    return hipGetLastError();
  }
  if (mx) return launch_mx(g, at, bt, ct, fp8_native, s);
  const bool a_kc = opA == AMP_OP_N, b_kc = opB == AMP_OP_T;
  if (at == AMP_E2M1X2) {
    const bool fast = aligned(A, 16) && aligned(B, 16) && lda % 16 == 0 && ldb % 16 == 0 &&
                      K % 64 == 0 && aligned(g.sA, 2) && aligned(g.sB, 2) && g.ldsA % 2 == 0 &&
                      g.ldsB % 2 == 0;
    if (!fast) return launch_generic<AMP_E2M1X2, AMP_E2M1X2>(g, true, true, ct, s);
    // full tiles, whole 256-K steps and 16-byte scale rows: codes to LDS by
    // direct loads, decoded per fragment
    constexpr int64_t kLim = int64_t(1) << 31;
    if (M % kBM == 0 && N % kBN == 0 && K % 256 == 0 && lda * kBM < kLim && ldb * kBN < kLim &&
        aligned(g.sA, 16) && aligned(g.sB, 16) && g.ldsA % 16 == 0 && g.ldsB % 16 == 0) {
      const dim3 grid(static_cast<unsigned>((M / kBM) * (N / kBN)));
      switch (ct) {
        case AMP_F32: gemm_mfma_d2l<AMP_E2M1X2, AMP_E2M1X2, true, true, kPFP4D, AMP_F32><<<grid, kThreads, 0, s>>>(g); break;
        case AMP_BF16: gemm_mfma_d2l<AMP_E2M1X2, AMP_E2M1X2, true, true, kPFP4D, AMP_BF16><<<grid, kThreads, 0, s>>>(g); break;
        default: gemm_mfma_d2l<AMP_E2M1X2, AMP_E2M1X2, true, true, kPFP4D, AMP_F16><<<grid, kThreads, 0, s>>>(g); break;
      }
      return hipGetLastError();
    }
    return launch_mfma<AMP_E2M1X2, AMP_E2M1X2, true, true, kPFP4>(g, ct, s);
  }
  if (at == AMP_E4M3 || at == AMP_E5M2) {
    const bool fast = aligned(A, 16) && aligned(B, 16) && lda % 16 == 0 && ldb % 16 == 0 &&
                      K % 16 == 0;
    if (at == AMP_E4M3 && bt == AMP_E4M3) return launch_f8<AMP_E4M3, AMP_E4M3>(g, fast, fp8_native, ct, s);
    if (at == AMP_E4M3) return launch_f8<AMP_E4M3, AMP_E5M2>(g, fast, fp8_native, ct, s);
    if (bt == AMP_E4M3) return launch_f8<AMP_E5M2, AMP_E4M3>(g, fast, fp8_native, ct, s);
    return launch_f8<AMP_E5M2, AMP_E5M2>(g, fast, fp8_native, ct, s);
  }
  // 16-bit: the vector path needs 16-byte aligned rows and the contiguous
  // extent of every operand a multiple of 8 elements
  bool fast = aligned(A, 16) && aligned(B, 16) && lda % 8 == 0 && ldb % 8 == 0;
  fast = fast && (a_kc ? K % 8 == 0 : M % 8 == 0) && (b_kc ? K % 8 == 0 : N % 8 == 0);
  if (at == AMP_BF16) return launch_16<AMP_BF16>(g, a_kc, b_kc, fast, ct, s);
  return launch_16<AMP_F16>(g, a_kc, b_kc, fast, ct, s);
}

hipError_t launch_gemm_blockwise(int64_t M, int64_t N, int64_t K, const void* A, int at,
                                 int64_t lda, const float* sA, int64_t ldsA, int a_block,
                                 const void* B, int bt, int64_t ldb, const float* sB,
                                 int64_t ldsB, int b_block, void* C, int ct, int64_t ldc,
                                 hipStream_t s) {
  BwArgs g{static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(B), C, M, N, K, lda, ldb,
           ldc, sA, sB, ldsA, ldsB, a_block, b_block};
  // matrix-core path: full 256x128 tiles, whole K-blocks, A's scales per row
  // (16-byte aligned scale rows), 32-bit buffer offsets
  constexpr int64_t kLim = int64_t(1) << 31;
  const bool fast = M % kBwBM == 0 && N % kBwBN == 0 && K % 128 == 0 && K > 0 && !a_block &&
                    aligned(A, 16) && aligned(B, 16) && lda % 16 == 0 && ldb % 16 == 0 &&
                    lda * kBwBM < kLim && ldb * kBwBN < kLim && aligned(sA, 16) && ldsA % 4 == 0 &&
                    ((K / 128) * ldsA + kBwBM) * 4 < kLim && bt == AMP_E4M3;
  if (at == AMP_E4M3 && bt == AMP_E4M3) return launch_bw_t<AMP_E4M3, AMP_E4M3>(g, fast, ct, s);
  if (at == AMP_E5M2 && bt == AMP_E4M3) return launch_bw_t<AMP_E5M2, AMP_E4M3>(g, fast, ct, s);
  if (at == AMP_E4M3) return launch_bw_t<AMP_E4M3, AMP_E5M2>(g, false, ct, s);
  return launch_bw_t<AMP_E5M2, AMP_E5M2>(g, false, ct, s);
}

}  // namespace amp
