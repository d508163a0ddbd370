// Fused NHWC implicit-GEMM convolution kernels for gfx950 (CDNA4) and the
// run / pack entry points of the C ABI.
//
// GEMM view (TensorFlow conv_grad_filter_ops.cc, Im2col: one patch row per
// output pixel (n, ho, wo), columns in (r, s, c) order; the filter viewed as
// [R*S*C, K] as in conv_ops_fused_int8.cc's GEMM special cases):
//   rows m = (n, ho, wo)       M  = N*Ho*Wo
//   cols k = output channel    K
//   reduction kk = (r, s, c)   Kg = R*S*C
// The patch matrix is never built: each lane gathers its 16-byte slice of a
// patch row straight from the NHWC input with a predicated load (taps in the
// padding read as zero), so padding costs no extra pass.
//
// Matrix-core mapping.  The 16x16 MFMA computes D[i][j] = sum_k A[i][k]B[k][j]
// with lane l supplying A row (l % 16) and B column (l % 16), each a 16-byte
// slice of k chosen by l / 16, and receiving D rows 4*(l/16) .. 4*(l/16)+3 of
// column l % 16.  We run the product transposed -- A = packed filter rows
// (output channels), B = patch rows (pixels) -- so a lane ends with outputs
// of ONE pixel.  The filter repack permutes the channel order inside each
// 64-channel block so those outputs are 16 CONSECUTIVE channels: the fused
// epilogue then reads its side input and writes y with one 16-byte access per
// lane, and a wave's 16 pixels x 64 channels of int8 are 1 KiB of contiguous
// NHWC.
//
// Per 16-byte chunk of the reduction each lane issues:
//   int8: 1 x v_mfma_i32_16x16x64_i8   (16 int8 per lane, exact int32 sums)
//   bf16: 1 x v_mfma_f32_16x16x32_bf16 (8 bf16 per lane, fp32 sums)
//   fp32: 4 x v_mfma_f32_16x16x4_f32   (4 fp32 per lane, one per instruction)
// Any permutation of the reduction index gives the same sum as long as A and
// B use the same one, which holds because both come from the same kk.
//
// Build with -ffp-contract=off: the int8 epilogue is specified operation by
// operation (scale, fused side multiply-add, bias, round half to even) and a
// contraction the compiler invents would change the int8 result.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>
#include <vector>

#include "plan.h"

namespace fconv {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;  // 4 waves of 64
constexpr int kTileM = 64;     // pixels per workgroup (16 per wave)
constexpr int kTileN = 64;     // output channels per workgroup

template <int DT> struct Dt;
template <> struct Dt<FCONV_INT8> {
  using T = int8_t;
  using Acc = i32x4;
  static constexpr int kChunk = 16;
};
template <> struct Dt<FCONV_BF16> {
  using T = uint16_t;  // raw bf16 bits
  using Acc = f32x4;
  static constexpr int kChunk = 8;
};
template <> struct Dt<FCONV_FP32> {
  using T = float;
  using Acc = f32x4;
  static constexpr int kChunk = 4;
};

__device__ inline i32x4 mma_chunk(i32x4 a, i32x4 b, i32x4 c,
                                  Dt<FCONV_INT8>*) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 mma_chunk(i32x4 a, i32x4 b, f32x4 c, Dt<FCONV_BF16>*) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
// Bit-cast the whole vector, then index: clang lowers a bit-cast of a single
// ext-vector element (e.g. __builtin_bit_cast(float, a.y)) to a load from the
// vector's base address, i.e. it silently reads element 0.
__device__ inline f32x4 mma_chunk(i32x4 a, i32x4 b, f32x4 c, Dt<FCONV_FP32>*) {
  const f32x4 af = __builtin_bit_cast(f32x4, a);
  const f32x4 bf = __builtin_bit_cast(f32x4, b);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(af.x, bf.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(af.y, bf.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(af.z, bf.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(af.w, bf.w, c, 0, 0, 0);
  return c;
}

// Output channel held by packed filter row p.  Within each 64-row block, row
// j*16 + a (j = 16-row MFMA tile, a = row inside it) holds channel
// 16*(a/4) + 4*j + a%4, so lane group g = a/4 of every tile covers channels
// 16g .. 16g+15 of the block.
__host__ __device__ inline int packed_row_channel(int p) {
  const int a = p & 15, j = (p >> 4) & 3;
  return (p & ~63) + 16 * (a >> 2) + 4 * j + (a & 3);
}

struct ConvArgs {
  const void* x;
  const void* wp;  // packed filter [Kp][KgP]
  const float* bias;
  const int8_t* side;
  const float* bn_gamma;
  const float* bn_beta;
  const float* bn_mean;
  const float* bn_var;
  void* y;
  float cis, sis, bn_eps;
  int32_t N, H, W, C, K, R, S, sh, sw, pt, pl, Ho, Wo;
  int32_t M, Kg, KgP;
  int32_t wrow_bytes;  // packed filter row stride: KgP * elem + 16 (zero pad)
  uint32_t x_bytes, y_bytes, side_bytes;  // buffer-descriptor extents
  uint32_t wp_bytes;                      // packed filter extent
  int32_t tiles;                          // ceil(M / 16) pixel tiles
  // m / Wo and q / Ho by multiply-high: q = (umulhi(n, mul) + (add ? n : 0)) >> shift
  uint32_t wo_mul, wo_add, wo_shift, ho_mul, ho_add, ho_shift;
  int32_t use_side, use_bias, use_bn, relu;
  const float* cis_vec;  // per-channel conv_input_scale [K], or null: cis for all
  int32_t cudnn7;        // int8 epilogue in the cuDNN 7 order
  int32_t act;           // float activation: 0 none, 1 ReLU, 2 leaky, 3 clipped, 4 clamp
  float act_alpha, act_beta;
  // Row-halo kernel: output rows per workgroup and rows of its first phase
  // (set by its launcher).
  int32_t halo_rows, halo_rows_a;
  // Full-size VALID GEMM: partial sums [gemm_splits][N][Kp] (4 bytes each) in
  // the workspace after the packed filter, k-steps per split, padded K.
  void* part;
  int32_t gemm_splits, gemm_kps, Kp;
};

// ------------------------------------------------------------ filter repack

// HWIO [R][S][C][K] (= [Kg][K]) -> packed [Kp] rows of KgP elements plus a
// 16-byte zero pad (row stride wrow_bytes, an odd multiple of 16 bytes), rows
// in the permuted channel order above, reduction contiguous, zero-filled past
// K and Kg.  One thread per 16-byte chunk of the packed filter.
template <int DT>
__global__ __launch_bounds__(256) void pack_filter_kernel(const void* __restrict__ w_,
                                                          void* __restrict__ wp_,
                                                          int32_t K, int32_t Kg,
                                                          int32_t KgP, int32_t Kp) {
  using T = typename Dt<DT>::T;
  constexpr int E = Dt<DT>::kChunk;
  const T* w = static_cast<const T*>(w_);
  T* wp = static_cast<T*>(wp_);
  const int chunks_per_row = KgP / E + 1;  // + the pad chunk
  const int64_t id = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (id >= static_cast<int64_t>(Kp) * chunks_per_row) return;
  const int p = static_cast<int>(id / chunks_per_row);
  const int q = static_cast<int>(id - static_cast<int64_t>(p) * chunks_per_row);
  const int ch = packed_row_channel(p);
  union {
    T e[E];
    i32x4 v;
  } u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int kk = q * E + e;
    u.e[e] = (ch < K && kk < Kg) ? w[static_cast<int64_t>(kk) * K + ch] : T(0);
  }
  *reinterpret_cast<i32x4*>(wp + static_cast<int64_t>(p) * (KgP + E) + q * E) = u.v;
}

// ---------------------------------------------------------------- epilogues

// Cache policy of output stores.  y is written once and never read back by
// the kernel.  Non-temporal (nt) instead of the default measured 0.3 us
// faster on the 3x3 int8 layer and 0.55 us on the 1x1.  Where a wave writes
// whole lines (int8 with 16 channels per lane: four lanes write 64
// contiguous bytes, a wave 16 pixels x 64 channels of contiguous NHWC), sc1
// (device-scope write-through) on top of nt measured faster again: 3x3 int8
// 8.26 -> 8.00 us, 1x1 6.67 -> 6.23, strided int8 (256-pixel tiles) 20.0 ->
// 18.6.  bf16 and fp32 tiles, whose waves write partial lines, were 3-8%
// slower with sc1 and keep nt (bf16) or the default (fp32).
constexpr int kStoreNT = 2;
constexpr int kStoreLines = 16 | kStoreNT;

__device__ inline __amdgpu_buffer_rsrc_t output_rsrc(const void* y, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(y), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  // gfx950 converts in hardware (v_cvt_pk_bf16_f32, two values per
  // instruction): round to nearest even, a NaN kept quiet with its sign and
  // top payload bits.  Measured identical, bit for bit, on all 2^32 inputs to
  // the integer form of the same rounding (add 0x7fff plus the kept lsb; a
  // NaN gets its quiet bit set), which it replaces.
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Side-input chunk of output pixel m, channels ch0 .. ch0+NCH-1 (zero past
// K), NCH = 16 or 8 (then in the low 8 bytes).
template <int NCH = 16>
__device__ inline i32x4 load_side_chunk(const ConvArgs& a, int m, int ch0, bool kvec) {
  const int8_t* side = a.side + static_cast<int64_t>(m) * a.K + ch0;
  if (kvec) {
    if constexpr (NCH == 16) return *reinterpret_cast<const i32x4*>(side);
    const i32x2 v = *reinterpret_cast<const i32x2*>(side);
    return i32x4{v.x, v.y, 0, 0};
  }
  union {
    int8_t b[16];
    i32x4 v;
  } s;
  s.v = i32x4{0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < NCH; ++e) s.b[e] = (ch0 + e < a.K) ? side[e] : int8_t(0);
  return s.v;
}

// int8: TensorFlow conv_ops_fused_int8.cc, BiasActivationOutputKernel (cuDNN 8
// order).  v[e] is the int32 accumulator of channel ch0 + e; side_chunk holds
// the int8 side input of the same NCH channels (ignored unless a.use_side).
// The bias of a lane's NCH channels (0 past K), loaded once per lane: loads
// issued after an output store would wait for it, as the compiler cannot rule
// out that they alias.
template <int NCH>
__device__ inline void load_bias(const ConvArgs& a, int ch0, bool kvec, float (&bias)[NCH]) {
#pragma unroll
  for (int e = 0; e < NCH; ++e) {
    const int ch = ch0 + e;
    bias[e] = (kvec || ch < a.K) ? a.bias[ch] : 0.0f;
  }
}

// The conv_input_scale of a lane's NCH channels: the per-channel vector
// (0 past K) or the scalar.
template <int NCH>
__device__ inline void load_scales(const ConvArgs& a, int ch0, bool kvec, float (&cis)[NCH]) {
#pragma unroll
  for (int e = 0; e < NCH; ++e) {
    const int ch = ch0 + e;
    cis[e] = a.cis_vec ? ((kvec || ch < a.K) ? a.cis_vec[ch] : 0.0f) : a.cis;
  }
}

template <int NCH = 16>
__device__ inline void epilogue_store_i8(const int32_t (&v)[NCH], const ConvArgs& a,
                                         int m, int ch0, bool kvec, i32x4 side_chunk,
                                         const float (&bias)[NCH], const float (&cis)[NCH]) {
  int8_t* y = static_cast<int8_t*>(a.y) + static_cast<int64_t>(m) * a.K + ch0;
  union {
    int8_t b[16];
    i32x4 v;
  } s, o;
  s.v = side_chunk;
  o.v = i32x4{0, 0, 0, 0};
  const float lo = a.relu ? 0.0f : -128.0f;
#pragma unroll
  for (int e = 0; e < NCH; ++e) {
    const float b = bias[e];
    float t = static_cast<float>(v[e]);        // int32 -> fp32, nearest even
    if (a.cudnn7) {
      // cuDNN 7 order: scale and bias in one fused multiply-add, then side.
      t = __builtin_fmaf(t, cis[e], b);
      if (a.use_side) t = __builtin_fmaf(static_cast<float>(s.b[e]), a.sis, t);
    } else {
      t = t * cis[e];                          // (1) scale
      if (a.use_side) t = __builtin_fmaf(static_cast<float>(s.b[e]), a.sis, t);  // (2)
      t = t + b;                               // (3) bias
    }
    t = __builtin_rintf(t);                    // round half to even
    t = __builtin_fminf(__builtin_fmaxf(t, lo), 127.0f);
    o.b[e] = static_cast<int8_t>(static_cast<int32_t>(t));
  }
  if (kvec) {
    if constexpr (NCH == 16)
      __builtin_amdgcn_raw_buffer_store_b128(
          o.v, output_rsrc(a.y, a.y_bytes),
          static_cast<uint32_t>(m) * static_cast<uint32_t>(a.K) + static_cast<uint32_t>(ch0), 0,
          kStoreLines);
    else
      __builtin_nontemporal_store(i32x2{o.v.x, o.v.y}, reinterpret_cast<i32x2*>(y));
  } else {
#pragma unroll
    for (int e = 0; e < NCH; ++e)
      if (ch0 + e < a.K) y[e] = o.b[e];
  }
}

template <int NCH = 16>
__device__ inline void epilogue_store_i8(const int32_t (&v)[NCH], const ConvArgs& a,
                                         int m, int ch0, bool kvec, i32x4 side_chunk) {
  float bias[NCH], cis[NCH];
  load_bias<NCH>(a, ch0, kvec, bias);
  load_scales<NCH>(a, ch0, kvec, cis);
  epilogue_store_i8<NCH>(v, a, m, ch0, kvec, side_chunk, bias, cis);
}

// bf16 / fp32: bias -> batch-norm inference -> ReLU (MIOpen's CBNA order).
// Per-channel values of the float epilogue for a lane's NCH channels, loaded
// (and the batch-norm scale computed) once per lane; zero for channels past
// K, whose outputs are never stored.
template <int NCH>
struct FloatEpiParams {
  float bias[NCH], mean[NCH], sc[NCH], beta[NCH];
  __device__ inline void load(const ConvArgs& a, int ch0, bool kvec) {
#pragma unroll
    for (int e = 0; e < NCH; ++e) {
      const int ch = ch0 + e;
      const bool live = kvec || ch < a.K;
      bias[e] = a.use_bias && live ? a.bias[ch] : 0.0f;
      const bool bn = a.use_bn && live;
      sc[e] = bn ? a.bn_gamma[ch] / __builtin_sqrtf(a.bn_var[ch] + a.bn_eps) : 0.0f;
      mean[e] = bn ? a.bn_mean[ch] : 0.0f;
      beta[e] = bn ? a.bn_beta[ch] : 0.0f;
    }
  }
};

template <int DT, int NCH>
__device__ inline void epilogue_store_float(const float (&v)[NCH], const ConvArgs& a,
                                            int m, int ch0, bool kvec,
                                            const FloatEpiParams<NCH>& P) {
  float t[NCH];
#pragma unroll
  for (int e = 0; e < NCH; ++e) {
    float x = v[e];
    if (a.use_bias) x = x + P.bias[e];
    if (a.use_bn) x = (x - P.mean[e]) * P.sc[e] + P.beta[e];
    switch (a.act) {  // uniform
      case 1: x = __builtin_fmaxf(x, 0.0f); break;
      case 2: x = x > 0.0f ? x : a.act_alpha * x; break;
      case 3: x = __builtin_fminf(__builtin_fmaxf(x, 0.0f), a.act_alpha); break;
      case 4: x = __builtin_fminf(__builtin_fmaxf(x, a.act_alpha), a.act_beta); break;
      default: break;
    }
    t[e] = x;
  }
  const int64_t off = static_cast<int64_t>(m) * a.K + ch0;
  if constexpr (DT == FCONV_FP32) {
    float* y = static_cast<float*>(a.y) + off;
    if (kvec) {
#pragma unroll
      for (int q = 0; q < NCH / 4; ++q)
        *reinterpret_cast<f32x4*>(y + 4 * q) = f32x4{t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]};
    } else {
#pragma unroll
      for (int e = 0; e < NCH; ++e)
        if (ch0 + e < a.K) y[e] = t[e];
    }
  } else {
    uint16_t* y = static_cast<uint16_t*>(a.y) + off;
    union {
      uint16_t h[16];
      i32x4 v[2];
    } o;
#pragma unroll
    for (int e = 0; e < NCH; ++e) o.h[e] = f32_to_bf16_rne(t[e]);
    if (kvec) {
#pragma unroll
      for (int q = 0; q < NCH / 8; ++q)
        __builtin_nontemporal_store(o.v[q], reinterpret_cast<i32x4*>(y) + q);
    } else {
#pragma unroll
      for (int e = 0; e < NCH; ++e)
        if (ch0 + e < a.K) y[e] = o.h[e];
    }
  }
}

template <int DT, int NCH = 16>
__device__ inline void epilogue_store_float(const float (&v)[NCH], const ConvArgs& a,
                                            int m, int ch0, bool kvec) {
  FloatEpiParams<NCH> P;
  P.load(a, ch0, kvec);
  epilogue_store_float<DT, NCH>(v, a, m, ch0, kvec, P);
}

// ------------------------------------------------------------ general conv

// One lane's 16-byte slice of a patch row: reduction elements kk0 .. kk0+E-1
// of output pixel (n, hbase, wbase).  kLoadChunk: the slice lies in one tap
// (C % E == 0); kLoadElem: element by element.
template <int DT, int MODE>
__device__ inline i32x4 gather_patch_chunk(const typename Dt<DT>::T* __restrict__ xn,
                                           const ConvArgs& a, bool mvalid, int hbase,
                                           int wbase, int kk0) {
  using T = typename Dt<DT>::T;
  constexpr int E = Dt<DT>::kChunk;
  if constexpr (MODE == kLoadChunk) {
    i32x4 r = {0, 0, 0, 0};
    if (mvalid && kk0 < a.Kg) {
      const int tap = kk0 / a.C;
      const int c = kk0 - tap * a.C;
      const int rr = tap / a.S;
      const int hi = hbase + rr;
      const int wi = wbase + (tap - rr * a.S);
      if (hi >= 0 && hi < a.H && wi >= 0 && wi < a.W)
        r = *reinterpret_cast<const i32x4*>(xn + (hi * a.W + wi) * a.C + c);
    }
    return r;
  } else {
    union {
      T e[E];
      i32x4 v;
    } u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int kk = kk0 + e;
      T val = T(0);
      if (mvalid && kk < a.Kg) {
        const int tap = kk / a.C;
        const int c = kk - tap * a.C;
        const int rr = tap / a.S;
        const int hi = hbase + rr;
        const int wi = wbase + (tap - rr * a.S);
        if (hi >= 0 && hi < a.H && wi >= 0 && wi < a.W) val = xn[(hi * a.W + wi) * a.C + c];
      }
      u.e[e] = val;
    }
    return u.v;
  }
}

// Workgroup = 4 waves = 64 pixels x 64 output channels; wave w owns pixels
// 16w .. 16w+15 of the tile.  Operands come straight from global memory (the
// packed filter stays hot in L1/L2 across the grid).  Grid: (ceil(M/64), Kp/64).
template <int DT, int MODE, bool KVEC>
__global__ __launch_bounds__(kThreads) void conv_general_kernel(ConvArgs a) {
  using T = typename Dt<DT>::T;
  using Acc = typename Dt<DT>::Acc;
  constexpr int E = Dt<DT>::kChunk;
  constexpr int KSTEP = 4 * E;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;    // reduction slice of this lane / channel group
  const int col = lane & 15;  // pixel within the wave's 16
  const int m = blockIdx.x * kTileM + wave * 16 + col;
  const bool mvalid = m < a.M;

  int n = 0, ho = 0, wo = 0;
  if (mvalid) {
    wo = m % a.Wo;
    const int t = m / a.Wo;
    ho = t % a.Ho;
    n = t / a.Ho;
  }
  const int hbase = ho * a.sh - a.pt;
  const int wbase = wo * a.sw - a.pl;
  const T* __restrict__ xn =
      static_cast<const T*>(a.x) + static_cast<int64_t>(n) * a.H * a.W * a.C;
  // Packed filter row of this lane in MFMA tile 0; tile j adds 16 rows.
  const T* __restrict__ wrow = reinterpret_cast<const T*>(
                                   static_cast<const char*>(a.wp) +
                                   static_cast<int64_t>(blockIdx.y * kTileN + col) *
                                       a.wrow_bytes) +
                               g * E;
  const int64_t tile_stride = static_cast<int64_t>(16) * (a.wrow_bytes / sizeof(T));

  // The epilogue's per-channel values and side chunk are loaded before the
  // main loop, so their latency overlaps it (on small layers the kernel is a
  // chain of memory round trips).
  const int ch0 = blockIdx.y * kTileN + 16 * g;
  const bool live = mvalid && ch0 < a.K;
  float bias[16], cis[16];
  i32x4 sc = {0, 0, 0, 0};
  FloatEpiParams<16> P;
  if constexpr (DT == FCONV_INT8) {
    if (live) {
      load_bias<16>(a, ch0, KVEC, bias);
      load_scales<16>(a, ch0, KVEC, cis);
      if (a.use_side) sc = load_side_chunk(a, m, ch0, KVEC);
    }
  } else {
    if (live) P.load(a, ch0, KVEC);
  }

  Acc acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = Acc{0, 0, 0, 0};

  if constexpr (MODE == kLoadTap) {
    // A whole k-step (4 chunks) lies in one tap: the tap loop is uniform.
    int kk = 0;
    for (int r = 0; r < a.R; ++r) {
      const int hi = hbase + r;
      const bool hok = mvalid && hi >= 0 && hi < a.H;
      for (int s = 0; s < a.S; ++s) {
        const int wi = wbase + s;
        const bool ok = hok && wi >= 0 && wi < a.W;
        const T* px = xn + (hi * a.W + wi) * a.C + g * E;
        for (int c0 = 0; c0 < a.C; c0 += KSTEP, kk += KSTEP) {
          i32x4 b = {0, 0, 0, 0};
          if (ok) b = *reinterpret_cast<const i32x4*>(px + c0);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const i32x4 w4 = *reinterpret_cast<const i32x4*>(wrow + j * tile_stride + kk);
            acc[j] = mma_chunk(w4, b, acc[j], static_cast<Dt<DT>*>(nullptr));
          }
        }
      }
    }
  } else {
    // Two k-steps per trip, so that both steps' gathers are in flight at
    // once (the second only while it lies inside the packed rows).
    for (int kk = 0; kk < a.KgP; kk += 2 * KSTEP) {
      const bool two = kk + KSTEP < a.KgP;  // uniform
      const i32x4 b0 = gather_patch_chunk<DT, MODE>(xn, a, mvalid, hbase, wbase, kk + g * E);
      const i32x4 b1 = gather_patch_chunk<DT, MODE>(xn, a, mvalid && two, hbase, wbase,
                                                    kk + KSTEP + g * E);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const i32x4 w4 = *reinterpret_cast<const i32x4*>(wrow + j * tile_stride + kk);
        acc[j] = mma_chunk(w4, b0, acc[j], static_cast<Dt<DT>*>(nullptr));
      }
      if (two) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const i32x4 w4 = *reinterpret_cast<const i32x4*>(wrow + j * tile_stride + kk + KSTEP);
          acc[j] = mma_chunk(w4, b1, acc[j], static_cast<Dt<DT>*>(nullptr));
        }
      }
    }
  }

  if (!live) return;
  if constexpr (DT == FCONV_INT8) {
    int32_t v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * j + i] = acc[j][i];
    epilogue_store_i8<16>(v, a, m, ch0, KVEC, sc, bias, cis);
  } else {
    float v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * j + i] = acc[j][i];
    epilogue_store_float<DT, 16>(v, a, m, ch0, KVEC, P);
  }
}

// ------------------------------------------------ resident-filter conv

typedef __attribute__((address_space(3))) void* lds_ptr_t;
constexpr int kBufferDword3 = 0x00020000;  // raw buffer descriptor, gfx9 family
constexpr uint32_t kOutOfRange = 0x80000000u;  // offset past every extent: reads 0

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kBufferDword3);
}

// Resident-filter kernel.  The workgroup's 64-channel slice of the packed
// filter (64 padded rows, contiguous in global memory) is copied into LDS
// with direct global->LDS 16-byte loads, so it crosses L2 once per workgroup
// and costs no registers.  Each wave owns 16*PT consecutive output pixels x 64
// channels: one LDS filter fragment feeds PT MFMAs and one patch fragment
// feeds 4.  Patch fragments are raw buffer loads kept D k-steps ahead of the
// MFMAs in a register ring; a tap that falls in the padding gets an offset
// past the buffer's extent and reads zeros, so the gather has no branches.
// The side input is loaded before the main loop and y is written with buffer
// stores (pixels past M fall outside the extent and are dropped).
// Requires C % (4 chunks) == 0 (a k-step never straddles a tap), K % 16 == 0
// and x, y below 2 GiB.
//
// The packed rows' stride is an odd multiple of 16 bytes, so the 16 rows one
// ds_read_b128 touches land in 16 different 16-byte bank groups.
constexpr int kRfBN = 64;

template <int DT, int PT, int D>
__global__ __launch_bounds__(kThreads) void conv_rf_kernel(ConvArgs a) {
  using T = typename Dt<DT>::T;
  using Acc = typename Dt<DT>::Acc;
  constexpr int E = Dt<DT>::kChunk;
  constexpr int KSTEP = 4 * E;
  constexpr int ES = static_cast<int>(sizeof(T));
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int col = lane & 15;
  const int RS = a.wrow_bytes;
  const int ch0 = blockIdx.y * kRfBN + 16 * g;

  // 1. Filter slice -> LDS: 64 * RS bytes = 4 * RS chunks of 16 bytes, i.e.
  //    RS / 16 wave-wide 1 KiB copies, spread over the 4 waves.
  {
    const char* src = static_cast<const char*>(a.wp) +
                      static_cast<int64_t>(blockIdx.y) * kRfBN * RS;
    const int copies = RS / 16;
    for (int i = wave; i < copies; i += 4)
      __builtin_amdgcn_global_load_lds(src + i * 1024 + lane * 16,
                                       (lds_ptr_t)(smem + i * 1024), 16, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. Pixels of this lane (one per pixel tile) and their patch origins.
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const int CB = a.C * ES;  // bytes per input pixel
  const int mbase = blockIdx.x * (4 * 16 * PT) + wave * (16 * PT) + col;
  int hb[PT], wb[PT], pbase[PT];
#pragma unroll
  for (int p = 0; p < PT; ++p) {
    const int m = mbase + 16 * p;
    const int mm = m < a.M ? m : 0;
    const int wo = mm % a.Wo;
    const int t = mm / a.Wo;
    const int ho = t % a.Ho;
    const int n = t / a.Ho;
    // A pixel past M gets an origin no tap can bring back into the image.
    hb[p] = m < a.M ? ho * a.sh - a.pt : -(1 << 20);
    wb[p] = wo * a.sw - a.pl;
    pbase[p] = n * a.H * a.W * CB + g * E * ES;
  }

  // 3. Side input of every pixel tile (zeros when unused: empty extent).
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.side, a.use_side ? a.side_bytes : 0u);
  i32x4 side_frag[PT];
#pragma unroll
  for (int p = 0; p < PT; ++p)
    side_frag[p] = __builtin_amdgcn_raw_buffer_load_b128(
        sr, static_cast<uint32_t>((mbase + 16 * p) * a.K + ch0), 0, 0);

  // 4. Patch-fragment ring: k-step ks -> tap (r, s), channel offset c0.
  const int cs = a.C / KSTEP;
  const int nks = a.R * a.S * cs;
  auto issue = [&](int ks, i32x4(&f)[PT]) {
    const int tap = ks / cs;
    const int c0b = (ks - tap * cs) * KSTEP * ES;
    const int r = tap / a.S;
    const int s = tap - r * a.S;
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int hi = hb[p] + r;
      const int wi = wb[p] + s;
      const bool ok = static_cast<unsigned>(hi) < static_cast<unsigned>(a.H) &&
                      static_cast<unsigned>(wi) < static_cast<unsigned>(a.W);
      const uint32_t off = ok ? static_cast<uint32_t>(pbase[p] + (hi * a.W + wi) * CB + c0b)
                              : kOutOfRange;
      f[p] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
    }
  };
  i32x4 ring[D][PT];
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < nks) issue(d, ring[d]);

  // The filter copy was issued before the PT side loads and the ring's loads;
  // vector-memory loads retire in order, so once at most that many remain
  // outstanding this wave's part of the copy has landed in LDS.
  {
    constexpr int after = PT * (D + 1);
    static_assert(after < 64, "vmcnt field is 6 bits");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((after & 15) | ((after >> 4) << 14) | (7 << 4) | (15 << 8));
    __syncthreads();
  }

  Acc acc[PT][4];
#pragma unroll
  for (int p = 0; p < PT; ++p)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[p][j] = Acc{0, 0, 0, 0};

  const char* arow = smem + col * RS + g * E * ES;
  for (int ks0 = 0; ks0 < nks; ks0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int ks = ks0 + d;
      if (ks < nks) {
        i32x4 af[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          af[j] = *reinterpret_cast<const i32x4*>(arow + j * 16 * RS + ks * KSTEP * ES);
#pragma unroll
        for (int p = 0; p < PT; ++p)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[p][j] = mma_chunk(af[j], ring[d][p], acc[p][j], static_cast<Dt<DT>*>(nullptr));
        if (ks + D < nks) issue(ks + D, ring[d]);
      }
    }
  }

  // 5. Fused epilogue and stores.
  if (ch0 >= a.K) return;
#pragma unroll
  for (int p = 0; p < PT; ++p) {
    const int m = mbase + 16 * p;
    if constexpr (DT == FCONV_INT8) {
      int32_t v[16];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[4 * j + i] = acc[p][j][i];
      if (m < a.M) epilogue_store_i8(v, a, m, ch0, true, side_frag[p]);
    } else {
      float v[16];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[4 * j + i] = acc[p][j][i];
      if (m < a.M) epilogue_store_float<DT>(v, a, m, ch0, true);
    }
  }
}

// ----------------------------------------------------------- tiled conv

// n / d for n < 2^31 with host-computed (mul, add, shift); see make_fast_div.
__device__ inline uint32_t fast_div(uint32_t n, uint32_t mul, uint32_t add, uint32_t shift) {
  return (__umulhi(n, mul) + (add ? n : 0u)) >> shift;
}

// LDS-tiled implicit GEMM for reductions too long to keep the filter slice
// resident (bf16 / fp32 256-channel layers, int8 strided layers).  Workgroup
// tile: 128 pixels x 128 output channels, 8 waves (two per SIMD, so one
// wave's fragment reads, copies and barrier waits overlap the other's MFMAs)
// in a 2 x 4 grid of 64 pixels x 32 channels.
// The reduction advances in stages of 128 bytes (one filter tap, 128 bytes of
// its channels; two MFMA k-steps).  A stage of the tile (128 pixel rows and
// 128 filter rows of 128 bytes) arrives by buffer->LDS copies: 32 copies of
// 1 KiB, 4 per wave, into one of four LDS stage buffers, three stages ahead
// of the one being computed (the copies' latency under load is about three
// stages' compute); taps in the padding and rows past M or Kp read
// zeros.  Row r holds its 16-byte chunk c at slot c ^ (r & 7): a copy of 8
// whole rows lands contiguously, and the 16 rows one fragment read touches
// spread over all slots (contention-free ds_read_b128).  Each wave does a
// 4 x 2 grid of 16x16 MFMAs per k-step: 6 fragment reads feed 8 MFMAs.  A
// wave holds two of the four 16-row MFMA tiles of a 64-row packed filter
// block, so each lane owns 8 consecutive output channels.
constexpr int kTileBM = 128, kTileBN = 128, kTileStage = 128;

constexpr int kTileThreads = 512;

__host__ __device__ constexpr int vmcnt_imm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

template <int DT, bool KVEC, bool DS, int BM>
__global__ __launch_bounds__(kTileThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void conv_tile_kernel(ConvArgs a) {
  static_assert(BM == 128 || BM == 64, "pixel rows per tile");
  // BM = 64 (grids with at most half as many 128-pixel tiles as CUs): waves
  // of 32 pixels x 32 channels, one pixel copy per wave per stage.
  constexpr int PH = BM / 64;            // pixel copies per wave per stage
  constexpr int PI = BM / 32;            // 16-pixel MFMA tiles per wave
  constexpr int CPS = PH + 2;            // copies per wave per stage
  constexpr int MPS = 2 * PI * 2;        // MFMAs per wave per stage
  constexpr int TB = (BM + kTileBN) * kTileStage;  // bytes of one stage
  using Acc = typename Dt<DT>::Acc;
  constexpr int E = Dt<DT>::kChunk;
  constexpr int ES = 16 / E;
  constexpr int SE = kTileStage / ES;  // reduction elements per stage
  // Four distinct arrays, so that reading one stage never waits for the
  // copies still in flight into the others.
  __shared__ __attribute__((aligned(1024))) char buf0[TB];
  __shared__ __attribute__((aligned(1024))) char buf1[TB];
  __shared__ __attribute__((aligned(1024))) char buf2[TB];
  __shared__ __attribute__((aligned(1024))) char buf3[TB];
  // Epilogue values, copied before stage 0: for float, the tile's 128
  // channels of bias, gamma, var, mean and beta, one 1 KiB slot each (512
  // bytes used); for int8, bias and the per-channel scale in the first two
  // slots and the tile's side input (BM pixels x 128 bytes) after them.
  __shared__ __attribute__((aligned(1024))) char epar[DT == FCONV_INT8 ? 2048 + BM * 128 : 5 * 1024];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // pixel half, 32-channel quarter
  const int g = lane >> 4, col = lane & 15;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.wp, a.wp_bytes);

  // Copy role: copy h (h < PH) of this wave covers pixel rows
  // 64h + 8*wave .. +7 and filter copy h (h < 2) the filter rows BM + the
  // same; lane l fills slot l & 7 of row 8*wave + 64h + (l >> 3), i.e. chunk
  // q = (l & 7) ^ ((l >> 3) & 7) of that row.
  const int r0 = 8 * wave + (lane >> 3);
  const int q = (lane & 7) ^ ((lane >> 3) & 7);
  int hb[2], wb[2], pbase[2];
  uint32_t wbase[2];
  const int RS = a.wrow_bytes;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int m = blockIdx.x * BM + r0 + 64 * h;
    const int mm = m < a.M ? m : 0;
    const uint32_t qq = fast_div(static_cast<uint32_t>(mm), a.wo_mul, a.wo_add, a.wo_shift);
    const int wo = mm - static_cast<int>(qq) * a.Wo;
    const uint32_t n = fast_div(qq, a.ho_mul, a.ho_add, a.ho_shift);
    const int ho = static_cast<int>(qq) - static_cast<int>(n) * a.Ho;
    hb[h] = m < a.M ? ho * a.sh - a.pt : -(1 << 20);
    wb[h] = wo * a.sw - a.pl;
    pbase[h] = static_cast<int>(n) * a.H * a.W * a.C * ES + q * 16;
    wbase[h] = static_cast<uint32_t>((blockIdx.y * kTileBN + r0 + 64 * h) * RS + q * 16);
  }

  // Packed row blockIdx.y*128 + wn*32 + 16j + 4g + v is channel
  // 64*(2*blockIdx.y + wn/2) + 16g + 8*(wn%2) + 4j + v: 8 consecutive
  // channels per lane.  The epilogue's loads (per-channel values, the four
  // side chunks) are issued here, before the first copy, so that they land
  // during the main loop (and no later than the first stage's copies).
  const int ch0 = blockIdx.y * kTileBN + (wn >> 1) * 64 + 16 * g + 8 * (wn & 1);
  FloatEpiParams<8> fpar;
  if constexpr (DT == FCONV_INT8) {
    // Wave 0 copies the bias, wave 1 the per-channel scales (if any), and
    // every wave two 1 KiB pieces of the side tile (8 pixels of 128 bytes
    // each: lane l takes chunk l % 8 of pixel l / 8), all before their stage
    // copies, so the waits for stage 0 cover them; zeros past K and M.
    const int cbase = blockIdx.y * kTileBN;
    if (wave < 2) {
      const float* src = wave == 0 ? a.bias : a.cis_vec;
      const __amdgpu_buffer_rsrc_t pr =
          make_rsrc(src, src ? static_cast<uint32_t>(a.K) * 4u : 0u);
      const uint32_t off = lane < 32 ? static_cast<uint32_t>((cbase + 4 * lane) * 4) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(pr, (lds_ptr_t)(epar + wave * 1024), 16, off, 0, 0, 0);
    }
    if (a.use_side) {
      const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.side, a.side_bytes);
#pragma unroll
      for (int h = 0; h < PH; ++h) {
        const int piece = wave + 8 * h;                    // pixels 8*piece .. +7
        const int m = blockIdx.x * BM + 8 * piece + (lane >> 3);
        const int c = cbase + 16 * (lane & 7);
        const uint32_t off = m < a.M && c < a.K ? static_cast<uint32_t>(m * a.K + c) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_ptr_t)(epar + 2048 + piece * 1024), 16, off,
                                                 0, 0, 0);
      }
    }
  } else {
    // Waves 0-4 copy one vector each, before their stage copies, so the
    // waits for stage 0 cover them (zeros past K and for an absent op).
    if (wave < 5) {
      const float* src = wave == 0 ? a.bias : wave == 1 ? a.bn_gamma : wave == 2 ? a.bn_var
                       : wave == 3 ? a.bn_mean : a.bn_beta;
      const bool use = wave == 0 ? a.use_bias != 0 : a.use_bn != 0;
      const __amdgpu_buffer_rsrc_t pr =
          make_rsrc(use ? src : nullptr, use ? static_cast<uint32_t>(a.K) * 4u : 0u);
      const uint32_t off =
          lane < 32 ? static_cast<uint32_t>((blockIdx.y * kTileBN + 4 * lane) * 4) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(pr, (lds_ptr_t)(epar + wave * 1024), 16, off, 0, 0, 0);
    }
  }

  const int nst = a.R * a.S * (a.C / SE);
  const int CB = a.C * ES;  // bytes of one tap's channels
  // Position of the next stage to copy: channel byte offset c0b inside tap
  // (r, s), advanced one stage per call (no divisions).
  int nx_st = 0, nx_c0b = 0, nx_r = 0, nx_s = 0;
  // This wave's 4 copies of the next stage (past the last stage: zeros).
  auto issue = [&](char* buf) {
    const int st = nx_st, c0b = nx_c0b, r = nx_r, s = nx_s;
    ++nx_st;
    nx_c0b += kTileStage;
    if (nx_c0b == CB) {
      nx_c0b = 0;
      if (++nx_s == a.S) {
        nx_s = 0;
        ++nx_r;
      }
    }
    const bool live = st < nst;
#pragma unroll
    for (int h = 0; h < PH; ++h) {
      const int hi = hb[h] + r, wi = wb[h] + s;
      const bool ok = live && static_cast<unsigned>(hi) < static_cast<unsigned>(a.H) &&
                      static_cast<unsigned>(wi) < static_cast<unsigned>(a.W);
      const uint32_t off =
          ok ? static_cast<uint32_t>(pbase[h] + (hi * a.W + wi) * a.C * ES + c0b) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (lds_ptr_t)(buf + (8 * wave + 64 * h) * kTileStage), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr, (lds_ptr_t)(buf + (BM + 8 * wave + 64 * h) * kTileStage), 16,
          live ? wbase[h] + st * kTileStage : kOutOfRange, 0, 0, 0);
  };

  Acc acc[PI][2];
#pragma unroll
  for (int i = 0; i < PI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = Acc{0, 0, 0, 0};

  // Fragment rows: pixel row wm*64 + 16i + col, filter row 128 + wn*32 +
  // 16j + col; both have (row & 7) == (col & 7).
  struct Frags {
    i32x4 pf[2][PI], ff[2][2];
  };
  auto read_frags = [&](const char* buf, Frags& f) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint32_t slot = static_cast<uint32_t>(((kk * 4 + g) ^ (col & 7)) * 16);
      const char* pl = buf + (wm * (BM / 2) + col) * kTileStage + slot;
      const char* fb = buf + (BM + wn * 32 + col) * kTileStage + slot;
#pragma unroll
      for (int i = 0; i < PI; ++i) f.pf[kk][i] = *reinterpret_cast<const i32x4*>(pl + i * 16 * kTileStage);
#pragma unroll
      for (int j = 0; j < 2; ++j) f.ff[kk][j] = *reinterpret_cast<const i32x4*>(fb + j * 16 * kTileStage);
    }
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < PI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = mma_chunk(f.ff[kk][j], f.pf[kk][i], acc[i][j], static_cast<Dt<DT>*>(nullptr));
  };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Step st computes stage st from fragments read during step st - 1 and
  // reads stage st + 1's fragments while its MFMAs run, so the matrix core
  // never waits for a stage's LDS reads.  Each wave first waits for its own
  // copies of stage st + 1 (stage st + 2's 4 may still be in flight), then a
  // plain s_barrier: LDS has no cache, so every wave's copies of stage st + 1
  // are visible after it, and every wave has consumed stage st - 1, whose
  // buffer the copies of stage st + 3 issued next reuse.  (__syncthreads()
  // would add a release fence that waits for all copies.)
  auto step = [&](const char* next, char* next3, const Frags& cur, Frags& nxt) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPS));
    barrier();
    issue(next3);  // stage + 3, into the buffer of the stage before this one
    read_frags(next, nxt);
    mma(cur);
    // Order: the fragment reads first (left alone, the scheduler sinks them
    // to the end of the step, and the next step's MFMAs wait on them), then
    // the copies spread between the MFMAs, so that a copy stalled on a busy
    // memory pipe does not hold the matrix core idle.
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (PI + 2), 0);  // DS read
#pragma unroll
    for (int q = 0; q < CPS; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, MPS / CPS, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read (the copy)
    }
    if constexpr (MPS % CPS != 0) __builtin_amdgcn_sched_group_barrier(0x008, MPS % CPS, 0);
    // Issue every MFMA before the next step's wait and barrier (otherwise
    // the scheduler hoists the barrier above them and the MFMAs queue behind
    // the barrier wait).
    __builtin_amdgcn_sched_barrier(0);
  };

  // Stage st lives in buffer st % 4.  Whole trips of four stages in the
  // loop (no exit in between, so the accumulators stay in place), the rest
  // after it.  Past the last stage the copies are zeros and the fragment
  // reads unused.
  issue(buf0);
  issue(buf1);
  issue(buf2);
  Frags fa, fb;
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * CPS));  // this wave's copies of stage 0
  barrier();
  read_frags(buf0, fa);
  int st = 0;
  if constexpr (DS) {
    // DS: two stages per barrier.  Every copy (stages st + 1 and st + 2) and
    // every LDS read has completed before it, then stages st + 3 and st + 4
    // are copied into the buffers of st - 1 and st (both read during the
    // previous double step), stage st is computed from cur while st + 1's
    // fragments are read, then st + 1 from them while st + 2's are read
    // into cur.
    auto dstep = [&](const char* b1, const char* b2, char* c3, char* c4)
        __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0);
      barrier();
      issue(c3);
      issue(c4);
      read_frags(b1, fb);
      mma(fa);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (PI + 2), 0);  // DS read
#pragma unroll
      for (int q = 0; q < 2 * CPS; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, MPS / (2 * CPS), 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read (the copy)
      }
      if constexpr (MPS % (2 * CPS) != 0)
        __builtin_amdgcn_sched_group_barrier(0x008, MPS % (2 * CPS), 0);
      __builtin_amdgcn_sched_barrier(0);
      read_frags(b2, fa);
      mma(fb);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (PI + 2), 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, MPS, 0);  // MFMA
      __builtin_amdgcn_sched_barrier(0);
    };
    for (; st + 4 <= nst; st += 4) {
      dstep(buf1, buf2, buf3, buf0);
      dstep(buf3, buf0, buf1, buf2);
    }
    if (st + 2 <= nst) {
      dstep(buf1, buf2, buf3, buf0);
      st += 2;
    }
    if (st < nst) mma(fa);  // the last stage, read by the double step before
  } else {
  for (; st + 4 <= nst; st += 4) {
    step(buf1, buf3, fa, fb);
    step(buf2, buf0, fb, fa);
    step(buf3, buf1, fa, fb);
    step(buf0, buf2, fb, fa);
  }
  if (st < nst) step(buf1, buf3, fa, fb);
  if (st + 1 < nst) step(buf2, buf0, fb, fa);
  if (st + 2 < nst) step(buf3, buf1, fa, fb);
  }
  __builtin_amdgcn_s_waitcnt(0);  // copies past the last stage (zeros) land before exit

  if (ch0 >= a.K) return;
  if constexpr (DT == FCONV_INT8) {
    // Per-channel values and side chunks from LDS (landed before the first
    // barrier).
    const int cl = ch0 - blockIdx.y * kTileBN;
    const float* eb = reinterpret_cast<const float*>(epar);
    float bias_l[8], cis_l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bias_l[e] = eb[cl + e];
      cis_l[e] = a.cis_vec ? eb[256 + cl + e] : a.cis;
    }
#pragma unroll
    for (int i = 0; i < PI; ++i) {
      const int p = wm * (BM / 2) + i * 16 + col;
      const int m = blockIdx.x * BM + p;
      if (m >= a.M) continue;
      int32_t v[8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * j + e] = acc[i][j][e];
      i32x4 sd = i32x4{0, 0, 0, 0};
      if (a.use_side) {
        const i32x2 w2 = *reinterpret_cast<const i32x2*>(epar + 2048 + p * 128 + cl);
        sd = i32x4{w2.x, w2.y, 0, 0};
      }
      epilogue_store_i8<8>(v, a, m, ch0, KVEC, sd, bias_l, cis_l);
    }
  } else {
    // Per-channel values from LDS (landed before the first barrier), with
    // the arithmetic of FloatEpiParams::load.
    const float* ep = reinterpret_cast<const float*>(epar) + (ch0 - blockIdx.y * kTileBN);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      fpar.bias[e] = a.use_bias ? ep[e] : 0.0f;
      fpar.sc[e] = a.use_bn ? ep[256 + e] / __builtin_sqrtf(ep[512 + e] + a.bn_eps) : 0.0f;
      fpar.mean[e] = a.use_bn ? ep[768 + e] : 0.0f;
      fpar.beta[e] = a.use_bn ? ep[1024 + e] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < PI; ++i) {
      const int m = blockIdx.x * BM + wm * (BM / 2) + i * 16 + col;
      if (m >= a.M) continue;
      float v[8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * j + e] = acc[i][j][e];
      epilogue_store_float<DT, 8>(v, a, m, ch0, KVEC, fpar);
    }
  }
}

// The tiled kernel with a copy role (int8 and bf16, 128- and 64-pixel tiles):
// 12 waves.  Waves 0-3, one per SIMD and started first, issue every
// buffer->LDS copy of a stage, BM/32 of pixel rows and 4 of filter rows each,
// three stages ahead, and the epilogue values' copies before stage 0.  Waves
// 4-11, two per SIMD, only read fragments and run MFMAs, as the 2 x 4 grid of
// the 8-wave kernel (BM/2 pixels x 32 channels each): no memory instruction,
// no copy arithmetic and no memory-count wait in their loop.  Step st reads
// stage st + 1's fragments while stage st's MFMAs run; before the barrier
// that ends it, the copy waves have issued stage st + 3 into the buffer of
// stage st - 1 and waited until only those copies are in flight (stage st + 2
// has landed), and the MFMA waves have waited for their reads.  The tile,
// stage layout, slot swizzle and epilogue are the 8-wave kernel's.  Measured
// (same box, graph replay): 26.2-26.3 -> 23.4-23.6 us on the 3x3 256-channel
// bf16 layer, 22.1 -> 20.3 (5x5 CBNA) and 22.4-22.6 -> 20.7-20.8 (7x7 stride-2
// CBNA, 64-pixel tiles), 19.3 -> 19.0 on the strided int8 layer pinned to
// 128-pixel tiles, same outputs bit for bit; fp32 153.3 against 154.3, so
// fp32 keeps the 8-wave kernel.  The copy waves also compute the batch-norm
// scale once per tile, and bf16 outputs are rounded by the hardware
// conversion: 23.6-23.75 -> 21.8 us and 20.3-20.4 -> 19.0-19.1 us (5x5 CBNA).
constexpr int kCwThreads = 768;

template <int DT, bool KVEC, int BM>
__global__ __launch_bounds__(kCwThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void conv_tile_cw_kernel(ConvArgs a) {
  static_assert(BM == 128 || BM == 64, "pixel rows per tile");
  constexpr int PI = BM / 32;  // 16-pixel MFMA tiles per MFMA wave
  constexpr int PC = BM / 32;  // pixel copies per copy wave per stage
  constexpr int CPW = PC + 4;  // copies per copy wave per stage
  constexpr int TB = (BM + kTileBN) * kTileStage;
  using Acc = typename Dt<DT>::Acc;
  constexpr int E = Dt<DT>::kChunk;
  constexpr int ES = 16 / E;
  constexpr int SE = kTileStage / ES;
  __shared__ __attribute__((aligned(1024))) char buf0[TB];
  __shared__ __attribute__((aligned(1024))) char buf1[TB];
  __shared__ __attribute__((aligned(1024))) char buf2[TB];
  __shared__ __attribute__((aligned(1024))) char buf3[TB];
  __shared__ __attribute__((aligned(1024))) char epar[DT == FCONV_INT8 ? 2048 + BM * 128 : 5 * 1024];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  const int nst = a.R * a.S * (a.C / SE);

  if (wave < 4) {
    const int e = wave;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.wp, a.wp_bytes);
    // Copy h of this wave: rows 8 (e + 4h) .. +7 of the pixel block and of
    // the filter block; lane l fills slot l & 7 of row 8 (e + 4h) + (l >> 3).
    const int q = (lane & 7) ^ ((lane >> 3) & 7);
    int hb[PC], wb[PC], pbase[PC];
    uint32_t wbase[4];
    const int RS = a.wrow_bytes;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int row = 8 * (e + 4 * h) + (lane >> 3);
      wbase[h] = static_cast<uint32_t>((blockIdx.y * kTileBN + row) * RS + q * 16);
    }
#pragma unroll
    for (int h = 0; h < PC; ++h) {
      const int row = 8 * (e + 4 * h) + (lane >> 3);
      const int m = blockIdx.x * BM + row;
      const int mm = m < a.M ? m : 0;
      const uint32_t qq = fast_div(static_cast<uint32_t>(mm), a.wo_mul, a.wo_add, a.wo_shift);
      const int wo = mm - static_cast<int>(qq) * a.Wo;
      const uint32_t n = fast_div(qq, a.ho_mul, a.ho_add, a.ho_shift);
      const int ho = static_cast<int>(qq) - static_cast<int>(n) * a.Ho;
      hb[h] = m < a.M ? ho * a.sh - a.pt : -(1 << 20);
      wb[h] = wo * a.sw - a.pl;
      pbase[h] = static_cast<int>(n) * a.H * a.W * a.C * ES + q * 16;
    }
    // Epilogue values before the stage copies, so that the wait for stage 0
    // covers them.
    if constexpr (DT == FCONV_INT8) {
      const int cbase = blockIdx.y * kTileBN;
      if (e < 2) {
        const float* src = e == 0 ? a.bias : a.cis_vec;
        const __amdgpu_buffer_rsrc_t pr = make_rsrc(src, src ? static_cast<uint32_t>(a.K) * 4u : 0u);
        const uint32_t off = lane < 32 ? static_cast<uint32_t>((cbase + 4 * lane) * 4) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pr, (lds_ptr_t)(epar + e * 1024), 16, off, 0, 0, 0);
      }
      if (a.use_side) {
        const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.side, a.side_bytes);
#pragma unroll
        for (int h = 0; h < PC; ++h) {
          const int piece = e + 4 * h;  // pixels 8 piece .. +7
          const int m = blockIdx.x * BM + 8 * piece + (lane >> 3);
          const int c = cbase + 16 * (lane & 7);
          const uint32_t off = m < a.M && c < a.K ? static_cast<uint32_t>(m * a.K + c) : kOutOfRange;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_ptr_t)(epar + 2048 + piece * 1024), 16, off, 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int v = e; v < 5; v += 4) {
        const float* src = v == 0 ? a.bias : v == 1 ? a.bn_gamma : v == 2 ? a.bn_var : v == 3 ? a.bn_mean : a.bn_beta;
        const bool use = v == 0 ? a.use_bias != 0 : a.use_bn != 0;
        const __amdgpu_buffer_rsrc_t pr = make_rsrc(use ? src : nullptr, use ? static_cast<uint32_t>(a.K) * 4u : 0u);
        const uint32_t off = lane < 32 ? static_cast<uint32_t>((blockIdx.y * kTileBN + 4 * lane) * 4) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pr, (lds_ptr_t)(epar + v * 1024), 16, off, 0, 0, 0);
      }
    }
    const int CB = a.C * ES;
    int nx_st = 0, nx_c0b = 0, nx_r = 0, nx_s = 0;
    auto issue = [&](char* buf) {
      const int st = nx_st, c0b = nx_c0b, r = nx_r, s = nx_s;
      ++nx_st;
      nx_c0b += kTileStage;
      if (nx_c0b == CB) {
        nx_c0b = 0;
        if (++nx_s == a.S) {
          nx_s = 0;
          ++nx_r;
        }
      }
      const bool live = st < nst;
#pragma unroll
      for (int h = 0; h < PC; ++h) {
        const int hi = hb[h] + r, wi = wb[h] + s;
        const bool ok = live && static_cast<unsigned>(hi) < static_cast<unsigned>(a.H) &&
                        static_cast<unsigned>(wi) < static_cast<unsigned>(a.W);
        const uint32_t off = ok ? static_cast<uint32_t>(pbase[h] + (hi * a.W + wi) * a.C * ES + c0b) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(buf + 8 * (e + 4 * h) * kTileStage), 16, off, 0, 0, 0);
      }
#pragma unroll
      for (int h = 0; h < 4; ++h)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(buf + (BM + 8 * (e + 4 * h)) * kTileStage), 16,
                                                 live ? wbase[h] + st * kTileStage : kOutOfRange, 0, 0, 0);
    };
    issue(buf0);
    issue(buf1);
    issue(buf2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPW));  // stages 0 and 1 (and the epilogue values) have landed
    barrier();
    if constexpr (DT != FCONV_INT8) {
      // The batch-norm scale of the tile's 128 channels, gamma / sqrt(var +
      // eps), computed once here in place of gamma: the MFMA waves read it
      // after their last barrier, and the first barrier below publishes it.
      if (a.use_bn && e < 2) {
        float* ep = reinterpret_cast<float*>(epar);
        const int c = 64 * e + lane;
        ep[256 + c] = ep[256 + c] / __builtin_sqrtf(ep[512 + c] + a.bn_eps);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    }
    // Step st: copy stage st + 3 into the buffer of stage st - 1, then wait
    // until only those 8 copies are in flight: stage st + 2 has landed
    // before the barrier that ends step st.
    int st = 0;
    for (; st + 4 <= nst; st += 4) {
      issue(buf3); __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPW)); barrier();
      issue(buf0); __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPW)); barrier();
      issue(buf1); __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPW)); barrier();
      issue(buf2); __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPW)); barrier();
    }
    if (st < nst) { issue(buf3); __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPW)); barrier(); }
    if (st + 1 < nst) { issue(buf0); __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPW)); barrier(); }
    if (st + 2 < nst) { issue(buf1); __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPW)); barrier(); }
    __builtin_amdgcn_s_waitcnt(0);  // copies past the last stage (zeros) land before exit
    return;
  }

  const int w = wave - 4;
  const int wm = w & 1, wn = w >> 1;  // pixel half, 32-channel quarter
  const int g = lane >> 4, col = lane & 15;
  const int ch0 = blockIdx.y * kTileBN + (wn >> 1) * 64 + 16 * g + 8 * (wn & 1);
  Acc acc[PI][2];
#pragma unroll
  for (int i = 0; i < PI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = Acc{0, 0, 0, 0};
  struct Frags {
    i32x4 pf[2][PI], ff[2][2];
  };
  auto read_frags = [&](const char* buf, Frags& f) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint32_t slot = static_cast<uint32_t>(((kk * 4 + g) ^ (col & 7)) * 16);
      const char* pl = buf + (wm * (BM / 2) + col) * kTileStage + slot;
      const char* fb = buf + (BM + wn * 32 + col) * kTileStage + slot;
#pragma unroll
      for (int i = 0; i < PI; ++i) f.pf[kk][i] = *reinterpret_cast<const i32x4*>(pl + i * 16 * kTileStage);
#pragma unroll
      for (int j = 0; j < 2; ++j) f.ff[kk][j] = *reinterpret_cast<const i32x4*>(fb + j * 16 * kTileStage);
    }
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < PI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = mma_chunk(f.ff[kk][j], f.pf[kk][i], acc[i][j], static_cast<Dt<DT>*>(nullptr));
  };
  // Step st: read stage st + 1's fragments, run stage st's MFMAs, then wait
  // for the reads (the buffer is recopied two steps later) and meet the copy
  // waves at the barrier.
  auto step = [&](const char* next, const Frags& cur, Frags& nxt) __attribute__((always_inline)) {
    read_frags(next, nxt);
    mma(cur);
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * (PI + 2), 0);  // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * PI, 0);        // MFMA
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    barrier();
  };
  Frags fa, fb;
  barrier();  // stages 0 and 1 have landed
  read_frags(buf0, fa);
  int st = 0;
  for (; st + 4 <= nst; st += 4) {
    step(buf1, fa, fb);
    step(buf2, fb, fa);
    step(buf3, fa, fb);
    step(buf0, fb, fa);
  }
  if (st < nst) step(buf1, fa, fb);
  if (st + 1 < nst) step(buf2, fb, fa);
  if (st + 2 < nst) step(buf3, fa, fb);

  if (ch0 >= a.K) return;
  if constexpr (DT == FCONV_INT8) {
    const int cl = ch0 - blockIdx.y * kTileBN;
    const float* eb = reinterpret_cast<const float*>(epar);
    float bias_l[8], cis_l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bias_l[e] = eb[cl + e];
      cis_l[e] = a.cis_vec ? eb[256 + cl + e] : a.cis;
    }
#pragma unroll
    for (int i = 0; i < PI; ++i) {
      const int p = wm * (BM / 2) + i * 16 + col;
      const int m = blockIdx.x * BM + p;
      if (m >= a.M) continue;
      int32_t v[8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * j + e] = acc[i][j][e];
      i32x4 sd = i32x4{0, 0, 0, 0};
      if (a.use_side) {
        const i32x2 w2 = *reinterpret_cast<const i32x2*>(epar + 2048 + p * 128 + cl);
        sd = i32x4{w2.x, w2.y, 0, 0};
      }
      epilogue_store_i8<8>(v, a, m, ch0, KVEC, sd, bias_l, cis_l);
    }
  } else {
    FloatEpiParams<8> fpar;
    const float* ep = reinterpret_cast<const float*>(epar) + (ch0 - blockIdx.y * kTileBN);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      fpar.bias[e] = a.use_bias ? ep[e] : 0.0f;
      fpar.sc[e] = a.use_bn ? ep[256 + e] : 0.0f;  // the scale, computed by the copy waves
      fpar.mean[e] = a.use_bn ? ep[768 + e] : 0.0f;
      fpar.beta[e] = a.use_bn ? ep[1024 + e] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < PI; ++i) {
      const int m = blockIdx.x * BM + wm * (BM / 2) + i * 16 + col;
      if (m >= a.M) continue;
      float v[8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * j + e] = acc[i][j][e];
      epilogue_store_float<DT, 8>(v, a, m, ch0, KVEC, fpar);
    }
  }
}

// Tall variant of the tiled kernel, for grids whose 128-pixel tiles would
// need a second round over the CUs while 256-pixel ones fit in one (the
// strided 56x56x128 layer: 392 tiles against 196).  Tile 256 pixels x 128
// channels, the same 8 waves as a 4 x 2 grid of 64 pixels x 64 channels
// (each lane ends with 16 consecutive channels of 4 pixels), the same
// 128-byte stages, slot swizzle and buffer->LDS copies (6 per wave per stage:
// 4 of pixel rows, 2 of filter rows), but three 48 KiB stage buffers with the
// copies two stages ahead: a stage's MFMAs take twice as long as in the
// 128-pixel tile, so one step covers the copies' latency, and a quarter fewer
// bytes are copied per MFMA.  Epilogue values (bias, scales, the float
// vectors) are copied to LDS before stage 0; the int8 side input is loaded
// from global memory at the end (LDS has no room for it).
constexpr int kTall = 256;
constexpr int kTallStage = (kTall + kTileBN) * kTileStage;  // 48 KiB

template <int DT, bool KVEC>
__global__ __launch_bounds__(kTileThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void conv_tile256_kernel(ConvArgs a) {
  using Acc = typename Dt<DT>::Acc;
  constexpr int E = Dt<DT>::kChunk;
  constexpr int ES = 16 / E;
  constexpr int SE = kTileStage / ES;       // reduction elements per stage
  constexpr int CPS = 6;                    // copies per wave per stage
  constexpr int MI = DT == FCONV_FP32 ? 4 : 1;  // MFMA instructions per chunk product
  constexpr int MPS = 32 * MI;              // MFMA instructions per wave per stage
  __shared__ __attribute__((aligned(1024))) char buf0[kTallStage];
  __shared__ __attribute__((aligned(1024))) char buf1[kTallStage];
  __shared__ __attribute__((aligned(1024))) char buf2[kTallStage];
  // int8: bias and per-channel scales of the tile's 128 channels (1 KiB slot
  // each, 512 bytes used); float: bias, gamma, var, mean, beta.
  __shared__ __attribute__((aligned(1024))) char epar[DT == FCONV_INT8 ? 2048 : 5 * 1024];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;  // 64-pixel quarter, 64-channel half
  const int g = lane >> 4, col = lane & 15;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.wp, a.wp_bytes);

  // Copy roles: pixel copy h (0..3) of this wave fills tile rows
  // 64h + 8*wave .. +7, filter copy h (0..1) filter rows 64h + 8*wave .. +7
  // (tile rows 256 + the same); lane l fills slot l & 7 of row r0 + 64h,
  // i.e. chunk q = (l & 7) ^ ((l >> 3) & 7) of that row.
  const int r0 = 8 * wave + (lane >> 3);
  const int q = (lane & 7) ^ ((lane >> 3) & 7);
  int hb[4], wb[4], pbase[4];
  uint32_t wbase[2];
  const int RS = a.wrow_bytes;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int m = blockIdx.x * kTall + r0 + 64 * h;
    const int mm = m < a.M ? m : 0;
    const uint32_t qq = fast_div(static_cast<uint32_t>(mm), a.wo_mul, a.wo_add, a.wo_shift);
    const int wo = mm - static_cast<int>(qq) * a.Wo;
    const uint32_t n = fast_div(qq, a.ho_mul, a.ho_add, a.ho_shift);
    const int ho = static_cast<int>(qq) - static_cast<int>(n) * a.Ho;
    hb[h] = m < a.M ? ho * a.sh - a.pt : -(1 << 20);
    wb[h] = wo * a.sw - a.pl;
    pbase[h] = static_cast<int>(n) * a.H * a.W * a.C * ES + q * 16;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
    wbase[h] = static_cast<uint32_t>((blockIdx.y * kTileBN + r0 + 64 * h) * RS + q * 16);

  // Packed row blockIdx.y*128 + wn*64 + 16j + 4g + v is channel
  // 128*blockIdx.y + 64*wn + 16g + 4j + v: 16 consecutive channels per lane.
  const int ch0 = blockIdx.y * kTileBN + wn * 64 + 16 * g;
  {
    // Epilogue vectors, before the first stage's copies (the wait for stage
    // 0 covers them); zeros past K and for an absent op.
    const int nv = DT == FCONV_INT8 ? 2 : 5;
    if (wave < nv) {
      const float* src;
      bool use;
      if constexpr (DT == FCONV_INT8) {
        src = wave == 0 ? a.bias : a.cis_vec;
        use = src != nullptr;
      } else {
        src = wave == 0 ? a.bias : wave == 1 ? a.bn_gamma : wave == 2 ? a.bn_var
            : wave == 3 ? a.bn_mean : a.bn_beta;
        use = wave == 0 ? a.use_bias != 0 : a.use_bn != 0;
      }
      const __amdgpu_buffer_rsrc_t pr =
          make_rsrc(use ? src : nullptr, use ? static_cast<uint32_t>(a.K) * 4u : 0u);
      const uint32_t off =
          lane < 32 ? static_cast<uint32_t>((blockIdx.y * kTileBN + 4 * lane) * 4) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(pr, (lds_ptr_t)(epar + wave * 1024), 16, off, 0, 0, 0);
    }
  }

  const int nst = a.R * a.S * (a.C / SE);
  const int CB = a.C * ES;  // bytes of one tap's channels
  int nx_st = 0, nx_c0b = 0, nx_r = 0, nx_s = 0;
  auto issue = [&](char* buf) __attribute__((always_inline)) {
    const int st = nx_st, c0b = nx_c0b, r = nx_r, s = nx_s;
    ++nx_st;
    nx_c0b += kTileStage;
    if (nx_c0b == CB) {
      nx_c0b = 0;
      if (++nx_s == a.S) {
        nx_s = 0;
        ++nx_r;
      }
    }
    const bool live = st < nst;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int hi = hb[h] + r, wi = wb[h] + s;
      const bool ok = live && static_cast<unsigned>(hi) < static_cast<unsigned>(a.H) &&
                      static_cast<unsigned>(wi) < static_cast<unsigned>(a.W);
      const uint32_t off =
          ok ? static_cast<uint32_t>(pbase[h] + (hi * a.W + wi) * a.C * ES + c0b) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (lds_ptr_t)(buf + (8 * wave + 64 * h) * kTileStage), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr, (lds_ptr_t)(buf + (kTall + 8 * wave + 64 * h) * kTileStage), 16,
          live ? wbase[h] + st * kTileStage : kOutOfRange, 0, 0, 0);
  };

  Acc acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = Acc{0, 0, 0, 0};

  // Fragment rows: pixel row wm*64 + 16i + col, filter row 256 + wn*64 +
  // 16j + col; both have (row & 7) == (col & 7).
  struct Frags {
    i32x4 pf[2][4], ff[2][4];
  };
  auto read_frags = [&](const char* buf, Frags& f) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint32_t slot = static_cast<uint32_t>(((kk * 4 + g) ^ (col & 7)) * 16);
      const char* pl = buf + (wm * 64 + col) * kTileStage + slot;
      const char* fb = buf + (kTall + wn * 64 + col) * kTileStage + slot;
#pragma unroll
      for (int i = 0; i < 4; ++i) f.pf[kk][i] = *reinterpret_cast<const i32x4*>(pl + i * 16 * kTileStage);
#pragma unroll
      for (int j = 0; j < 4; ++j) f.ff[kk][j] = *reinterpret_cast<const i32x4*>(fb + j * 16 * kTileStage);
    }
  };
  auto mma = [&](const Frags& f) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = mma_chunk(f.ff[kk][j], f.pf[kk][i], acc[i][j], static_cast<Dt<DT>*>(nullptr));
  };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Step st: wait for this wave's copies of stage st + 1 (issued one step
  // earlier; nothing later is in flight), a plain barrier (LDS has no cache:
  // every wave's copies of stage st + 1 are visible after it, and every wave
  // has read stage st - 1's fragments), copy stage st + 2 into stage
  // st - 1's buffer, read stage st + 1's fragments while stage st's MFMAs
  // run.
  auto step = [&](const char* next, char* next2, const Frags& cur, Frags& nxt)
      __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    barrier();
    issue(next2);
    read_frags(next, nxt);
    mma(cur);
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // DS read
#pragma unroll
    for (int c = 0; c < CPS; ++c) {
      __builtin_amdgcn_sched_group_barrier(0x008, MPS / CPS, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read (the copy)
    }
    if constexpr (MPS % CPS != 0) __builtin_amdgcn_sched_group_barrier(0x008, MPS % CPS, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Stage st lives in buffer st % 3: whole trips of three stages, then the
  // rest.  Past the last stage the copies are zeros and the fragment reads
  // unused.
  issue(buf0);
  issue(buf1);
  Frags fa, fb;
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(CPS));  // this wave's copies of stage 0 (and the vectors)
  barrier();
  read_frags(buf0, fa);
  int st = 0;
  for (; st + 6 <= nst; st += 6) {
    step(buf1, buf2, fa, fb);
    step(buf2, buf0, fb, fa);
    step(buf0, buf1, fa, fb);
    step(buf1, buf2, fb, fa);
    step(buf2, buf0, fa, fb);
    step(buf0, buf1, fb, fa);
  }
  // The rest (0..5 stages), starting from buffer 0 with fa current.
  if (st < nst) step(buf1, buf2, fa, fb);
  if (st + 1 < nst) step(buf2, buf0, fb, fa);
  if (st + 2 < nst) step(buf0, buf1, fa, fb);
  if (st + 3 < nst) step(buf1, buf2, fb, fa);
  if (st + 4 < nst) step(buf2, buf0, fa, fb);
  __builtin_amdgcn_s_waitcnt(0);  // copies past the last stage (zeros) land before exit

  if (ch0 >= a.K) return;
  const int cl = ch0 - blockIdx.y * kTileBN;
  const float* ep = reinterpret_cast<const float*>(epar) + cl;
  if constexpr (DT == FCONV_INT8) {
    float bias_l[16], cis_l[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      bias_l[e] = ep[e];
      cis_l[e] = a.cis_vec ? ep[256 + e] : a.cis;
    }
    i32x4 sd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = blockIdx.x * kTall + wm * 64 + i * 16 + col;
      sd[i] = a.use_side && m < a.M ? load_side_chunk<16>(a, m, ch0, KVEC) : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = blockIdx.x * kTall + wm * 64 + i * 16 + col;
      if (m >= a.M) continue;
      int32_t v[16];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * j + e] = acc[i][j][e];
      epilogue_store_i8<16>(v, a, m, ch0, KVEC, sd[i], bias_l, cis_l);
    }
  } else {
    FloatEpiParams<16> fpar;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      fpar.bias[e] = a.use_bias ? ep[e] : 0.0f;
      fpar.sc[e] = a.use_bn ? ep[256 + e] / __builtin_sqrtf(ep[512 + e] + a.bn_eps) : 0.0f;
      fpar.mean[e] = a.use_bn ? ep[768 + e] : 0.0f;
      fpar.beta[e] = a.use_bn ? ep[1024 + e] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = blockIdx.x * kTall + wm * 64 + i * 16 + col;
      if (m >= a.M) continue;
      float v[16];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * j + e] = acc[i][j][e];
      epilogue_store_float<DT, 16>(v, a, m, ch0, KVEC, fpar);
    }
  }
}

// ------------------------------------------------------- streaming conv

// int8 requantisation, cuDNN 8 order (TensorFlow conv_ops_fused_int8.cc,
// BiasActivationOutputKernel): (float)acc * cis, + side * sis as one fused
// multiply-add, + bias, each an fp32 operation.  Round half to even and clip
// are done together: adding 1.5 * 2^23 rounds t to the nearest integer (ties
// to even) into the low mantissa bits, exactly for |t| < 2^22, and monotonically
// beyond, where the clip saturates anyway; a med3 against the two biased
// bounds clips, and the low byte of the result's bit pattern is then the int8
// value (two's complement).  Checked exhaustively over every finite fp32 t.
// `lo_b` / `hi_b` are 1.5*2^23 + (ReLU ? 0 : -128) and 1.5*2^23 + 127.
constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23

// Scheduling pattern of one k-step chunk: each of its MFMAs followed by up
// to 4 VALU instructions, which issue while the matrix core works on the
// MFMA (a single wave per SIMD issues in order), then the chunk's fragment
// load.
template <int NMFMA = 4>
__device__ inline void interleave_mfma_valu() {
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
  }
}

// Low bytes of two / of two pairs packed with v_perm_b32.
__device__ inline uint32_t pack_pair(uint32_t lo_val, uint32_t hi_val) {
  return __builtin_amdgcn_perm(hi_val, lo_val, 0x0c0c0400u);  // [lo.b0, hi.b0, 0, 0]
}
__device__ inline uint32_t pack_word(uint32_t lo_pair, uint32_t hi_pair) {
  return __builtin_amdgcn_perm(hi_pair, lo_pair, 0x05040100u);  // [lo.b0, lo.b1, hi.b0, hi.b1]
}


// One lane's NOUT/4 packed output words with a single buffer store.
template <int NOUT>
__device__ inline void store_words(const uint32_t (&w)[NOUT / 4], __amdgpu_buffer_rsrc_t yr,
                                   uint32_t off) {
  if constexpr (NOUT == 16)
    __builtin_amdgcn_raw_buffer_store_b128(
        i32x4{static_cast<int32_t>(w[0]), static_cast<int32_t>(w[1]),
              static_cast<int32_t>(w[2]), static_cast<int32_t>(w[3])},
        yr, off, 0, kStoreLines);
  else
    __builtin_amdgcn_raw_buffer_store_b64(
        i32x2{static_cast<int32_t>(w[0]), static_cast<int32_t>(w[1])}, yr, off, 0, kStoreLines);
}

// Requantisation of a lane's NOUT (8 or 16) outputs, organised by stage so
// that a streaming kernel can spread it over the k-steps of the next tile:
// a stage runs one operation on 8 or 16 outputs at once, so the values are
// independent chains and every operation's input was produced a whole k-step
// earlier (VALU latency stays hidden).  Stages, in order:
//   cvt   8 accumulators out of the accumulation registers -> fp32 (NOUT/8 stages)
//   mul   * conv_input_scale
//   side  8 outputs: side byte -> fp32, fused multiply-add by sis (NOUT/8
//         stages; none without a side input)
//   bias  + bias
//   magic + 1.5 * 2^23 (round half to even)
//   med3  clip
//   pack  byte packing into NOUT/4 words
template <bool SIDE, int NOUT, bool ORDER7 = false>
struct EpiI8 {
  static constexpr int kCvt = NOUT / 8;
  static constexpr int kSide = SIDE ? NOUT / 8 : 0;
  static constexpr int kStages = kCvt + 1 + kSide + 4;
  float t[NOUT];
  uint32_t w[NOUT / 4];

  __device__ inline void stage(int st, const i32x4 (&acc)[NOUT / 4], i32x4 side_chunk,
                               const float (&bias)[NOUT], const float (&cis)[NOUT], float sis,
                               float lo_b, float hi_b) {
    union {
      int8_t b[16];
      i32x4 v;
    } sd;
    sd.v = side_chunk;
    if (st < kCvt) {
#pragma unroll
      for (int e = 8 * st; e < 8 * st + 8; ++e) t[e] = static_cast<float>(acc[e / 4][e % 4]);
      return;
    }
    st -= kCvt;
    if (st == 0) {
#pragma unroll
      for (int e = 0; e < NOUT; ++e) {
        if constexpr (ORDER7)
          t[e] = __builtin_fmaf(t[e], cis[e], bias[e]);  // cuDNN 7: scale and bias fused
        else
          t[e] = t[e] * cis[e];
      }
      return;
    }
    st -= 1;
    if (st < kSide) {
#pragma unroll
      for (int e = 8 * st; e < 8 * st + 8; ++e)
        t[e] = __builtin_fmaf(static_cast<float>(sd.b[e]), sis, t[e]);
      return;
    }
    st -= kSide;
    switch (st) {
      case 0:
        if constexpr (!ORDER7) {
#pragma unroll
          for (int e = 0; e < NOUT; ++e) t[e] = t[e] + bias[e];
        }
        break;
      case 1:
#pragma unroll
        for (int e = 0; e < NOUT; ++e) t[e] = t[e] + kRoundMagic;
        break;
      case 2:
#pragma unroll
        for (int e = 0; e < NOUT; ++e) t[e] = __builtin_amdgcn_fmed3f(t[e], lo_b, hi_b);
        break;
      default:
#pragma unroll
        for (int j = 0; j < NOUT / 4; ++j)
          w[j] = pack_word(pack_pair(__builtin_bit_cast(uint32_t, t[4 * j]),
                                     __builtin_bit_cast(uint32_t, t[4 * j + 1])),
                           pack_pair(__builtin_bit_cast(uint32_t, t[4 * j + 2]),
                                     __builtin_bit_cast(uint32_t, t[4 * j + 3])));
        break;
    }
  }
  // Keep the values produced so far in registers at this point of the
  // instruction stream (the arithmetic has no memory effects and would
  // otherwise be sunk to the store).
  __device__ inline void pin() {
#pragma unroll
    for (int i = 0; i < NOUT; i += 8)
      asm volatile("" : "+v"(t[i]), "+v"(t[i + 1]), "+v"(t[i + 2]), "+v"(t[i + 3]),
                   "+v"(t[i + 4]), "+v"(t[i + 5]), "+v"(t[i + 6]), "+v"(t[i + 7]));
#pragma unroll
    for (int j = 0; j < NOUT / 4; ++j) asm volatile("" : "+v"(w[j]));
  }
};

// Whole int8 epilogue of one tile for this lane's pixel and NOUT channels,
// written with one buffer store; an out-of-range offset drops it.
template <bool SIDE, int NOUT, bool ORDER7 = false>
__device__ inline void stream_epilogue_i8(const i32x4 (&acc)[NOUT / 4], i32x4 side_chunk,
                                          const float (&bias)[NOUT], const float (&cis)[NOUT],
                                          float sis,
                                          float lo_b, float hi_b, __amdgpu_buffer_rsrc_t yr,
                                          uint32_t off) {
  EpiI8<SIDE, NOUT, ORDER7> ep;
#pragma unroll
  for (int st = 0; st < EpiI8<SIDE, NOUT, ORDER7>::kStages; ++st)
    ep.stage(st, acc, side_chunk, bias, cis, sis, lo_b, hi_b);
  store_words<NOUT>(ep.w, yr, off);
}

// Streaming kernel for int8 layers with a short reduction: R x S taps of CS
// k-steps (64 channels each).  Persistent: one workgroup per CU of 4 "pixel
// waves", each walking every 4th 16-pixel tile of the workgroup's range.
// With KSPLIT = 2 a pixel wave is a pair of waves that split the 64-channel
// filter slice (32 channels and 8 outputs per lane each, two waves per
// SIMD); with KSPLIT = 1 one wave holds all 64 channels (16 outputs per
// lane, one wave per SIMD).  The filter slice stays in registers for the
// whole kernel.  Workgroup ranges are grouped by XCD so neighbouring tiles,
// which share input rows, share an L2.  Per tile, the patch fragments of all
// k-steps are buffer loads issued two tiles ahead; a tap outside the image
// gets an offset past the extent and reads zeros.  Offsets use 24-bit
// multiplies (every operand and product here is far below 2^24 / 2^31).
template <int R, int S, int CS, bool SIDE, int KSPLIT, bool ORDER7>
__global__ __launch_bounds__(256 * KSPLIT) __attribute__((amdgpu_waves_per_eu(KSPLIT, KSPLIT)))
void conv_stream_i8_kernel(ConvArgs a) {
  constexpr int NKS = R * S * CS;
  constexpr int NOUT = 16 / KSPLIT;  // outputs (channels) per lane
  constexpr int NJ = 4 / KSPLIT;     // 16-row MFMA tiles per wave
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kh = wave % KSPLIT;  // which channels of the slice
  const int pw = wave / KSPLIT;  // tiles pw, pw + 4, ... of the workgroup's range
  const int g = lane >> 4;
  const int col = lane & 15;
  const int ch0 = blockIdx.y * 64 + 16 * g + NOUT * kh;  // this lane's NOUT channels

  const int G = gridDim.x;
  const int bx = blockIdx.x;
  const int b = (G % 8 == 0) ? (bx % 8) * (G / 8) + bx / 8 : bx;
  const int t_begin = b * a.tiles / G;  // b * tiles < 2^31 (checked at plan time)
  const int t_end = (b + 1) * a.tiles / G;
  const int n_tiles = t_end - t_begin - pw > 0 ? (t_end - t_begin - pw + 3) / 4 : 0;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.side, SIDE ? a.side_bytes : 0u);
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(a.y, a.y_bytes);

  const int CB = a.C;          // bytes per input pixel
  const int WCB = a.W * CB;    // bytes per input row
  const int HWCB = a.H * WCB;  // bytes per image

  // Tap offsets relative to the tile pixel's patch origin (uniform).
  int delta[NKS];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int c = 0; c < CS; ++c) delta[(r * S + s) * CS + c] = r * WCB + s * CB + c * 64;

  // Buffer offsets of tile k's patch fragments (past the extent when the tap
  // falls outside the image or the tile outside this pair's range).
  auto offsets = [&](int k, uint32_t(&o)[NKS]) {
    const int t = t_begin + pw + 4 * k;
    const uint32_t m = static_cast<uint32_t>(t * 16 + col);
    const bool live = static_cast<unsigned>(k) < static_cast<unsigned>(n_tiles) &&
                      m < static_cast<uint32_t>(a.M);
    const uint32_t q = fast_div(m, a.wo_mul, a.wo_add, a.wo_shift);
    const int wo = static_cast<int>(m) - __mul24(static_cast<int>(q), a.Wo);
    const uint32_t n = fast_div(q, a.ho_mul, a.ho_add, a.ho_shift);
    const int ho = static_cast<int>(q) - __mul24(static_cast<int>(n), a.Ho);
    const int hb = __mul24(ho, a.sh) - a.pt;
    const int wb = __mul24(wo, a.sw) - a.pl;
    const int base = __mul24(static_cast<int>(n), HWCB) + __mul24(hb, WCB) +
                     __mul24(wb, CB) + g * 16;
    bool rok[R], cok[S];
#pragma unroll
    for (int r = 0; r < R; ++r)
      rok[r] = live && static_cast<unsigned>(hb + r) < static_cast<unsigned>(a.H);
#pragma unroll
    for (int s = 0; s < S; ++s)
      cok[s] = static_cast<unsigned>(wb + s) < static_cast<unsigned>(a.W);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int c = 0; c < CS; ++c) {
          const int ks = (r * S + s) * CS + c;
          o[ks] = (rok[r] && cok[s]) ? static_cast<uint32_t>(base + delta[ks]) : kOutOfRange;
        }
  };
  auto issue = [&](int k, i32x4(&f)[NKS]) {
    uint32_t o[NKS];
    offsets(k, o);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) f[ks] = __builtin_amdgcn_raw_buffer_load_b128(xr, o[ks], 0, 0);
  };
  // Output (and side-input) offset of tile k for this lane, or out of range.
  auto out_off = [&](int k) -> uint32_t {
    const int m = (t_begin + pw + 4 * k) * 16 + col;
    const bool ok = static_cast<unsigned>(k) < static_cast<unsigned>(n_tiles) &&
                    m < a.M && ch0 < a.K;
    return ok ? static_cast<uint32_t>(__mul24(m, a.K) + ch0) : kOutOfRange;
  };
  auto issue_side = [&](int k) -> i32x4 {
    if constexpr (SIDE) {
      if constexpr (NOUT == 16) return __builtin_amdgcn_raw_buffer_load_b128(sr, out_off(k), 0, 0);
      const i32x2 v = __builtin_amdgcn_raw_buffer_load_b64(sr, out_off(k), 0, 0);
      return i32x4{v.x, v.y, 0, 0};
    }
    return i32x4{0, 0, 0, 0};
  };

  // The first two tiles' patch fragments and side inputs are issued first,
  // so their latency overlaps the filter staging below.
  const i32x4 zero4 = i32x4{0, 0, 0, 0};
  i32x4 bA[NKS], bB[NKS];
  issue(0, bA);
  issue(1, bB);
  i32x4 sB = issue_side(-1);  // tile -1: out of range, reads zeros
  i32x4 sA = issue_side(0);

  // The 64-channel filter slice crosses L2 once per workgroup: a direct
  // global->LDS copy of its 64 padded rows, then every wave reads the
  // fragments of its rows for all k-steps into registers.  The bias of this
  // lane's channels comes in with buffer loads (channels past K read 0).
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int RS = a.wrow_bytes;
  {
    const char* src = static_cast<const char*>(a.wp) + static_cast<int64_t>(blockIdx.y) * 64 * RS;
    for (int i = wave; i < RS / 16; i += 4 * KSPLIT)
      __builtin_amdgcn_global_load_lds(src + i * 1024 + lane * 16,
                                       (lds_ptr_t)(smem + i * 1024), 16, 0, 0);
  }
  const __amdgpu_buffer_rsrc_t br = make_rsrc(a.bias, static_cast<uint32_t>(a.K) * 4u);
  float bias[NOUT];
#pragma unroll
  for (int q = 0; q < NOUT / 4; ++q) {
    const f32x4 v = __builtin_bit_cast(
        f32x4, __builtin_amdgcn_raw_buffer_load_b128(br, static_cast<uint32_t>((ch0 + 4 * q) * 4), 0, 0));
    bias[4 * q] = v.x;
    bias[4 * q + 1] = v.y;
    bias[4 * q + 2] = v.z;
    bias[4 * q + 3] = v.w;
  }
  float cis[NOUT];
  if (a.cis_vec) {
    const __amdgpu_buffer_rsrc_t cr = make_rsrc(a.cis_vec, static_cast<uint32_t>(a.K) * 4u);
#pragma unroll
    for (int q = 0; q < NOUT / 4; ++q) {
      const f32x4 v = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, static_cast<uint32_t>((ch0 + 4 * q) * 4), 0, 0));
      cis[4 * q] = v.x;
      cis[4 * q + 1] = v.y;
      cis[4 * q + 2] = v.z;
      cis[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < NOUT; ++e) cis[e] = a.cis;
  }
  const float sis = a.sis;
  const float lo_b = kRoundMagic + (a.relu ? 0.0f : -128.0f), hi_b = kRoundMagic + 127.0f;
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt = expcnt = lgkmcnt = 0
  __syncthreads();
  i32x4 Wf[NKS][NJ];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      Wf[ks][j] = *reinterpret_cast<const i32x4*>(smem + ((NJ * kh + j) * 16 + col) * RS +
                                                  ks * 64 + g * 16);

  i32x4 accA[NJ], accB[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) accB[j] = zero4;

  // One half of a loop trip, software-pipelined by hand: the MFMAs of the
  // tile in bX (into accX) are split by k-step into NKS chunks; each chunk
  // also issues that k-step's refill load for tile k_load and runs its share
  // of the epilogue stages of the previous tile (accY, side sY).  A
  // scheduling barrier closes each chunk.
  auto half = [&](i32x4(&bX)[NKS], i32x4(&accX)[NJ], const i32x4(&accY)[NJ], i32x4 sY,
                  int k_load, uint32_t off_prev) {
    uint32_t o[NKS];
    offsets(k_load, o);
    EpiI8<SIDE, NOUT, ORDER7> ep;
#pragma unroll
    for (int j = 0; j < NOUT / 4; ++j) ep.w[j] = 0u;
    constexpr int NS = EpiI8<SIDE, NOUT, ORDER7>::kStages;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        accX[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Wf[ks][j], bX[ks],
                                                        ks == 0 ? zero4 : accX[j], 0, 0, 0);
      bX[ks] = __builtin_amdgcn_raw_buffer_load_b128(xr, o[ks], 0, 0);
      // Epilogue stages [ceil(ks*NS/NKS), ceil((ks+1)*NS/NKS)) in this chunk.
#pragma unroll
      for (int st = (ks * NS + NKS - 1) / NKS; st < ((ks + 1) * NS + NKS - 1) / NKS; ++st)
        ep.stage(st, accY, sY, bias, cis, sis, lo_b, hi_b);
      ep.pin();
      interleave_mfma_valu<NJ>();
      __builtin_amdgcn_sched_barrier(0);
    }
    store_words<NOUT>(ep.w, yr, off_prev);
  };

  // Two tiles per trip and no exit in between, so both halves see the same
  // memory-operation history: half A computes tile k and finishes tile k-1,
  // half B computes tile k+1 and finishes tile k.  A tile past the pair's
  // range loads zeros and its store is dropped.
  int k = 0;
  for (; k < n_tiles; k += 2) {
    half(bA, accA, accB, sB, k + 2, out_off(k - 1));
    sB = issue_side(k + 1);
    half(bB, accB, accA, sA, k + 3, out_off(k));
    sA = issue_side(k + 2);
  }
  stream_epilogue_i8<SIDE, NOUT, ORDER7>(accB, sB, bias, cis, sis, lo_b, hi_b, yr, out_off(k - 1));
}

// ------------------------------------------------------------- row-halo int8
//
// Stride-1 int8 convolution over 64 input channels (one 64-byte k-step per
// filter tap) for short reductions such as 3x3x64.  A workgroup owns
// `halo_rows` consecutive output rows (flattened n*Ho + ho) and one 64-channel
// slice of the filter, split into two phases of rows: phase A is the first
// two rows, phase B the rest.  Loads are buffer->LDS copies: the filter slice and, for
// each phase, each distinct input row of the phase's footprint (zero rows and
// zero columns for the padding come from out-of-range buffer offsets, which
// read as zero).  Copies issue at a limited rate per CU, so the MFMA waves
// copy only the filter slice and phase A's rows and start computing as soon
// as those land, while the epilogue waves copy the bias and phase B's rows
// (each phase stages into its own LDS array, so reading one does not wait
// for copies into another).  B fragments are read from LDS, so no tile waits
// on device memory.  The side input streams in during the steps instead:
// each epilogue wave copies the 1 KiB side tile of its own tile two steps
// ahead into a three-slot ring and waits for it with a fixed vmcnt (its
// copies and stores alternate, and complete in issue order), so phase B's
// rows are not queued behind side data.
//
// Each input row lives in a 4 KiB slot: pixel X (halo column, X = input
// column + left pad) holds its four 16-byte channel chunks at positions
// 4X + (c ^ ((X >> 1) & 3)); with that swizzle a wave reading 16 consecutive
// pixels x one chunk per lane group runs at the contention-free ds_read_b128
// rate for any starting pixel.  A side tile uses the same swizzle over its
// 16 pixels.  Slot of tap row r for phase row j of image n:
// j + r + (R-1)*(n - n0), n0 = the phase's first image; consecutive output
// rows of one image share R-1 input rows, and each image change skips R-1
// slots so that rows of different images never collide.
//
// Waves 0-3 (one per SIMD) are MFMA waves: each walks every 4th 16-pixel
// tile of a phase with the whole 64-channel filter slice in registers and
// hands its int32 accumulators through LDS to epilogue wave 4-7 on the same
// SIMD, which requantises, adds the side input and stores.  The requantisation
// costs about as much SIMD time as the contraction; a VALU-only wave next to an
// MFMA-only wave overlaps the two, which a single wave doing both cannot.
// Steps are separated by workgroup barriers; the hand-off is double-buffered.
constexpr int kHaloSlot = 4096;
constexpr int kHaloRowsA = 2;       // output rows of phase A
constexpr int kHaloSlotsA = 6;      // input-row slots of phase A (two rows, up to two images)
constexpr int kHaloSlotsB = 9;      // input-row slots of phase B
constexpr int kHaloSideRing = 3;   // side-tile slots per epilogue wave
constexpr int kHaloThreads = 512;

__device__ inline uint32_t halo_pos(int x, int c) {
  return static_cast<uint32_t>(4 * x + (c ^ ((x >> 1) & 3)));
}

// Rows [p0, p1) of one phase.
struct HaloPhase {
  int p0, p1, n0, ho0, nslots, npx, ntile;
};

__device__ inline HaloPhase halo_phase(const ConvArgs& a, int p0, int p1, int R) {
  HaloPhase h;
  h.p0 = p0;
  h.p1 = p1;
  if (p1 <= p0) {
    h.n0 = h.ho0 = h.nslots = h.npx = h.ntile = 0;
    return h;
  }
  h.n0 = static_cast<int>(fast_div(static_cast<uint32_t>(p0), a.ho_mul, a.ho_add, a.ho_shift));
  const int n_last =
      static_cast<int>(fast_div(static_cast<uint32_t>(p1 - 1), a.ho_mul, a.ho_add, a.ho_shift));
  h.ho0 = p0 - h.n0 * a.Ho;
  h.nslots = (p1 - p0) + (R - 1) * (n_last - h.n0 + 1);
  h.npx = (p1 - p0) * a.Wo;
  h.ntile = (h.npx + 15) >> 4;
  return h;
}

// s_waitcnt vmcnt(min(n, 15)) (expcnt and lgkmcnt not waited on); waiting
// for fewer outstanding operations than allowed is always safe.
__device__ inline void wait_vmcnt_at_most(int n) {
  switch (n < 15 ? n : 15) {
#define FCONV_VMWAIT(k)                         \
  case k:                                       \
    __builtin_amdgcn_s_waitcnt(0x0f70 | (k));   \
    break;
    FCONV_VMWAIT(0) FCONV_VMWAIT(1) FCONV_VMWAIT(2) FCONV_VMWAIT(3) FCONV_VMWAIT(4)
    FCONV_VMWAIT(5) FCONV_VMWAIT(6) FCONV_VMWAIT(7) FCONV_VMWAIT(8) FCONV_VMWAIT(9)
    FCONV_VMWAIT(10) FCONV_VMWAIT(11) FCONV_VMWAIT(12) FCONV_VMWAIT(13) FCONV_VMWAIT(14)
    default:
      __builtin_amdgcn_s_waitcnt(0x0f70 | 15);
      break;
#undef FCONV_VMWAIT
  }
}

// Tail of the int8 requantisation of one tile in the epilogue wave, from
// t = (float)acc * cis (cuDNN 8 order) or t = fmaf((float)acc, cis, bias)
// (cuDNN 7 order), which the MFMA wave computed: the side input's fused
// multiply-add, the bias (cuDNN 8), then round half to even and clip, packed
// into four words.  With ReLU the rounding and the lower clip are those of
// v_cvt_pk_u8_f32, which rounds half to even and saturates to [0, 255]
// (checked on gfx950 over ties, their neighbours and out-of-range values):
// after t = min(t, 127) it gives clip(rint(t), 0, 127) in one instruction
// per output, packing included.  Without ReLU the 1.5 * 2^23 rounding and
// med3 clip of EpiI8.
template <bool SIDE, bool ORDER7, bool RELU>
__device__ inline void halo_epilogue_tail(float (&t)[16], i32x4 side_chunk,
                                          const float (&bias)[16], float sis, float lo_b,
                                          float hi_b, uint32_t (&w)[4]) {
  union {
    int8_t b[16];
    i32x4 v;
  } sd;
  sd.v = side_chunk;
  if constexpr (SIDE) {
#pragma unroll
    for (int e = 0; e < 16; ++e) t[e] = __builtin_fmaf(static_cast<float>(sd.b[e]), sis, t[e]);
  }
  if constexpr (!ORDER7) {
#pragma unroll
    for (int e = 0; e < 16; ++e) t[e] = t[e] + bias[e];
  }
  if constexpr (RELU) {
#pragma unroll
    for (int e = 0; e < 16; ++e) t[e] = __builtin_fminf(t[e], 127.0f);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t v = __builtin_amdgcn_cvt_pk_u8_f32(t[4 * j], 0u, 0u);
      v = __builtin_amdgcn_cvt_pk_u8_f32(t[4 * j + 1], 1u, v);
      v = __builtin_amdgcn_cvt_pk_u8_f32(t[4 * j + 2], 2u, v);
      w[j] = __builtin_amdgcn_cvt_pk_u8_f32(t[4 * j + 3], 3u, v);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      t[e] = __builtin_amdgcn_fmed3f(t[e] + kRoundMagic, lo_b, hi_b);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = pack_word(pack_pair(__builtin_bit_cast(uint32_t, t[4 * j]),
                                 __builtin_bit_cast(uint32_t, t[4 * j + 1])),
                       pack_pair(__builtin_bit_cast(uint32_t, t[4 * j + 2]),
                                 __builtin_bit_cast(uint32_t, t[4 * j + 3])));
  }
}

template <int R, int S, bool SIDE, bool ORDER7, bool RELU>
__global__ __launch_bounds__(kHaloThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void conv_halo_i8_kernel(ConvArgs a) {
  constexpr int NKS = R * S;
  constexpr int RSB = NKS * 64 + 16;  // packed filter row bytes
  __shared__ __attribute__((aligned(16))) char wlds[64 * RSB];
  __shared__ __attribute__((aligned(256))) char xa[kHaloSlotsA * kHaloSlot];
  __shared__ __attribute__((aligned(256))) char xb[kHaloSlotsB * kHaloSlot];
  __shared__ __attribute__((aligned(256))) char sring[SIDE ? 4 * kHaloSideRing * 1024 : 16];
  // Accumulator hand-off, per MFMA wave and step parity: chunk q (accumulator
  // tile q, 4 int32) of lane l at q * 1024 + 16 * l.
  __shared__ __attribute__((aligned(256))) char accb[4 * 2 * 4096];
  // The slice's 64 bias values (a copy's 64 lanes write 1 KiB: lanes past
  // the 16 that carry values write zeros).
  __shared__ __attribute__((aligned(16))) float blds[256];

  const int lane = threadIdx.x & 63;
  // readfirstlane: the wave index (and so the role) is uniform per wave.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool mfma_role = wave < 4;  // waves 0-3 MFMA, 4-7 epilogue (same SIMDs)
  const int m = wave & 3;           // tiles m, m + 4, ... of each phase
  const int g = lane >> 4;
  const int col = lane & 15;
  const int ch0 = blockIdx.y * 64 + 16 * g;

  const int G = gridDim.x;
  const int bx = blockIdx.x;
  const int b = (G % 8 == 0) ? (bx % 8) * (G / 8) + bx / 8 : bx;
  const int rows_total = a.N * a.Ho;
  const int g0 = b * a.halo_rows;
  if (g0 >= rows_total) return;  // uniform per workgroup
  const int g1 = min(g0 + a.halo_rows, rows_total);
  const int ga = min(g0 + a.halo_rows_a, g1);
  const HaloPhase PA = halo_phase(a, g0, ga, R);
  const HaloPhase PB = halo_phase(a, ga, g1, R);
  const int sA = (PA.ntile + 3) >> 2;  // steps of each phase (4 tiles per step)
  const int sB = (PB.ntile + 3) >> 2;

  // The MFMA waves turn their accumulators into t = (float)acc * cis (or
  // fmaf((float)acc, cis, bias) in the cuDNN 7 order) before the hand-off,
  // so they need the scales (and, cuDNN 7, the bias) of their lane's 16
  // channels: register loads issued here, which land with the copies the
  // MFMA waves wait for before the first barrier.  K is a multiple of 16.
  float cis_r[16], bias_r[16];
  if (mfma_role) {
    const bool live = ch0 < a.K;
#pragma unroll
    for (int e = 0; e < 16; ++e) {  // the [K] vectors are only 4-byte aligned
      cis_r[e] = a.cis_vec && live ? a.cis_vec[ch0 + e] : a.cis;
      bias_r[e] = ORDER7 && live ? a.bias[ch0 + e] : 0.0f;
    }
  }

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.side, SIDE ? a.side_bytes : 0u);
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(a.y, a.y_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.wp, a.wp_bytes);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(a.bias, static_cast<uint32_t>(a.K) * 4u);

  // ---- buffer->LDS copies of 1 KiB.  Nothing is loaded into registers:
  // a register load issued among the copies could only be waited for together
  // with all of them.
  auto copy_rows = [&](const HaloPhase& P, char* xbuf, int k) {
    const int sigma = k >> 2;
    // image segment e holding slot sigma: phase rows [js, je) of image n0+e
    // own slots [js + (R-1)e, je + (R-1)(e+1)).
    int e = 0, js = 0;
    int je = min(P.p1 - P.p0, a.Ho - P.ho0);
    while (sigma >= je + (R - 1) * (e + 1)) {
      ++e;
      js = je;
      je = min(P.p1 - P.p0, je + a.Ho);
    }
    const int n = P.n0 + e;
    const int hi = (e == 0 ? P.ho0 : 0) - a.pt + (sigma - js - (R - 1) * e);
    const int pos = (k & 3) * 64 + lane;  // position inside the 4 KiB slot
    const int X = pos >> 2;
    const int c = (pos & 3) ^ ((X >> 1) & 3);
    const int wi = X - a.pl;
    const bool ok = static_cast<unsigned>(hi) < static_cast<unsigned>(a.H) &&
                    static_cast<unsigned>(wi) < static_cast<unsigned>(a.W);
    const uint32_t src = ok ? static_cast<uint32_t>(((n * a.H + hi) * a.W + wi) * 64 + c * 16)
                            : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        xr, (lds_ptr_t)(xbuf + sigma * kHaloSlot + (k & 3) * 1024), 16, src, 0, 0, 0);
  };
  // Side tile of this epilogue wave's tile at (global) step t into ring slot
  // t % 3; past the last step it reads nothing (an out-of-range copy keeps
  // the wave's count of memory operations per step fixed).
  auto copy_side = [&](int t) {
    const bool in_a = t < sA;
    const int ls = in_a ? t : t - sA;
    const int npx = in_a ? PA.npx : PB.npx;
    const int pbase = (in_a ? PA.p0 : PB.p0) * a.Wo;
    const int pp = (m + 4 * ls) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((pp >> 1) & 3);
    const int ch = blockIdx.y * 64 + 16 * c;
    const bool ok = t < sA + sB && pp < npx && ch < a.K;
    const uint32_t src = ok ? static_cast<uint32_t>((pbase + pp) * a.K + ch) : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        sr, (lds_ptr_t)(sring + (m * kHaloSideRing + t % kHaloSideRing) * 1024), 16, src, 0, 0, 0);
  };

  {
    // All eight waves copy the filter slice and phase A's rows, then wait
    // for their own copies: the first step needs nothing else.
    const int e1 = RSB / 16;  // 64 rows of RSB bytes = RSB/16 KiB
    const int e2 = e1 + 4 * PA.nslots;
    for (int i = wave; i < e2; i += 8) {
      if (i < e1) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, (lds_ptr_t)(wlds + i * 1024), 16,
            static_cast<uint32_t>(blockIdx.y * 64 * RSB + i * 1024 + lane * 16), 0, 0, 0);
      } else {
        copy_rows(PA, xa, i - e1);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
  // Every wave has waited for the copies the next step reads before it
  // arrives, and LDS has no cache, so a plain s_barrier publishes them.
  // (__syncthreads() would add a release fence, which waits for every
  // outstanding copy.)
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  barrier();  // the filter slice and phase A's rows have landed
  if (!mfma_role) {
    // Epilogue waves copy the side tiles of their first two steps, the bias
    // and phase B's rows, after the first barrier so that the first step's
    // data has the memory system to itself.  They wait for the side tiles
    // and the bias before the barrier that ends step 0, and for phase B's
    // rows before the barrier that ends the last phase-A step.
    if constexpr (SIDE) {
      copy_side(0);
      copy_side(1);
    }
    const int e3 = 1 + 4 * PB.nslots;
    for (int i = m; i < e3; i += 4) {
      if (i == 0) {
        const uint32_t off = lane < 16 ? static_cast<uint32_t>((blockIdx.y * 64 + 4 * lane) * 4)
                                       : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_ptr_t)blds, 16, off, 0, 0, 0);
      } else {
        copy_rows(PB, xb, i - 1);
      }
    }
  }

  if (mfma_role) {
    i32x4 Wf[NKS][4];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        Wf[ks][j] = *reinterpret_cast<const i32x4*>(wlds + (j * 16 + col) * RSB + ks * 64 + g * 16);
    const i32x4 zero4 = i32x4{0, 0, 0, 0};

    // One phase of MFMA steps.  Step ls computes tile m + 4*ls (lanes past
    // the phase's pixels read the last pixel; their results are never
    // stored) and hands its accumulators to the epilogue wave of this SIMD.
    auto mfma_phase = [&](const HaloPhase& P, const char* xbuf, int steps, int step0) {
      if (steps == 0) return;
      // LDS addresses of the tile of step ls for this lane: tap (r, s) is
      // ad[s] + r * kHaloSlot.
      auto tile_addr = [&](int ls, uint32_t(&ad)[S]) {
        const int p = min((m + 4 * ls) * 16 + col, P.npx - 1);
        const int j = static_cast<int>(fast_div(static_cast<uint32_t>(p), a.wo_mul, a.wo_add, a.wo_shift));
        const int wo = p - j * a.Wo;
        const int n = static_cast<int>(fast_div(static_cast<uint32_t>(P.p0 + j), a.ho_mul, a.ho_add, a.ho_shift));
        const uint32_t base = static_cast<uint32_t>((j + (R - 1) * (n - P.n0)) * kHaloSlot);
#pragma unroll
        for (int s = 0; s < S; ++s) ad[s] = base + 16u * halo_pos(wo + s, g);
      };
      auto frag = [&](uint32_t addr) -> i32x4 {
        return *reinterpret_cast<const i32x4*>(xbuf + addr);
      };
      i32x4 bf[NKS];
      {
        uint32_t ad[S];
        tile_addr(0, ad);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) bf[ks] = frag(ad[ks % S] + (ks / S) * kHaloSlot);
      }
      for (int ls = 0; ls < steps; ++ls) {
        // The next step's fragments are refilled k-step by k-step as soon
        // as this step's MFMAs have consumed them.
        uint32_t ad[S];
        tile_addr(ls + 1 < steps ? ls + 1 : ls, ad);
        i32x4 acc[4];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Wf[ks][j], bf[ks],
                                                           ks == 0 ? zero4 : acc[j], 0, 0, 0);
          bf[ks] = frag(ad[ks % S] + (ks / S) * kHaloSlot);
        }
        // Keep each refill next to its k-step's MFMAs so that its latency
        // hides under the remaining ones (left alone, the scheduler moves
        // every read to the end of the step).
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
        // First steps of the requantisation, each an fp32 operation of the
        // specification: t = (float)acc (nearest even), then * cis, or one
        // fused multiply-add with the bias in the cuDNN 7 order.
        char* dst = accb + (m * 2 + ((step0 + ls) & 1)) * 4096 + 16 * lane;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 t4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float t = static_cast<float>(acc[j][e]);
            t4[e] = ORDER7 ? __builtin_fmaf(t, cis_r[4 * j + e], bias_r[4 * j + e])
                           : t * cis_r[4 * j + e];
          }
          *reinterpret_cast<f32x4*>(dst + j * 1024) = t4;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): hand-off written
        barrier();
      }
    };
    // Phase A always has a step; phase B's rows were published by the
    // barrier that ends step 0, before phase B's first fragments are read.
    mfma_phase(PA, xa, sA, 0);
    mfma_phase(PB, xb, sB, sA);
    barrier();  // the epilogue waves' last step
  } else {
    // Step 0 (the MFMA waves compute the first tiles): wait for this wave's
    // copies before the barrier that publishes them to the other waves; no
    // output has been stored yet.  Phase B's first fragments are read after
    // the barrier that ends the last phase-A step, so with two phase-A steps
    // this wave's row copies (issued last) may stay in flight one step
    // longer: they are waited for at the end of epilogue step 0, where the
    // step's store and (with a side input) the copy of side tile 2 have been
    // issued since.
    const int rows_m = ((1 + 4 * PB.nslots - m + 3) >> 2) - ((1 - m + 3) >> 2);
    if (sA >= 2)
      wait_vmcnt_at_most(rows_m);
    else
      __builtin_amdgcn_s_waitcnt(0);
    barrier();
    float bias[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) bias[e] = blds[16 * g + e];
    const float sis = a.sis;
    const float lo_b = kRoundMagic + (a.relu ? 0.0f : -128.0f), hi_b = kRoundMagic + 127.0f;
    auto epi_phase = [&](const HaloPhase& P, int steps, int step0) {
      for (int ls = 0; ls < steps; ++ls) {
        const int t = step0 + ls;
        const char* src = accb + (m * 2 + (t & 1)) * 4096 + 16 * lane;
        i32x4 acc[4];
        const int p = (m + 4 * ls) * 16 + col;
        i32x4 sd = i32x4{0, 0, 0, 0};
        if constexpr (SIDE) {
          // The side tile of step t >= 2 was copied at step t - 2, after
          // that step's store; the store of step t - 1 and the copy of step
          // t + 1 have been issued since, so vmcnt(2) covers it (earlier
          // tiles landed before the first step).  The reads are issued in
          // one block with that wait: a compiler-generated read of the ring
          // would wait for every copy in flight into it.
          const char* sp = sring + (m * kHaloSideRing + t % kHaloSideRing) * 1024 +
                           16u * halo_pos(col, g);
          const uint32_t acc_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)src));
          const uint32_t side_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)sp));
          asm volatile(
              "s_waitcnt vmcnt(2)\n\t"
              "ds_read_b128 %0, %5\n\t"
              "ds_read_b128 %1, %5 offset:1024\n\t"
              "ds_read_b128 %2, %5 offset:2048\n\t"
              "ds_read_b128 %3, %5 offset:3072\n\t"
              "ds_read_b128 %4, %6\n\t"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(acc[0]), "=&v"(acc[1]), "=&v"(acc[2]), "=&v"(acc[3]), "=&v"(sd)
              : "v"(acc_addr), "v"(side_addr)
              : "memory");
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j] = *reinterpret_cast<const i32x4*>(src + j * 1024);
        }
        const bool ok = p < P.npx && ch0 < a.K;
        const uint32_t off = ok ? static_cast<uint32_t>((P.p0 * a.Wo + p) * a.K + ch0) : kOutOfRange;
        // The hand-off holds t as fp32 bits (bit-cast whole vectors: a
        // bit-cast of one ext-vector element reads element 0).
        float tv[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 f = __builtin_bit_cast(f32x4, acc[j]);
#pragma unroll
          for (int e = 0; e < 4; ++e) tv[4 * j + e] = f[e];
        }
        uint32_t w[4];
        halo_epilogue_tail<SIDE, ORDER7, RELU>(tv, sd, bias, sis, lo_b, hi_b, w);
        store_words<16>(w, yr, off);
        if constexpr (SIDE) copy_side(t + 2);  // into the slot step t - 1 read
        if (t == 0 && sA >= 2) __builtin_amdgcn_s_waitcnt(SIDE ? 0x0f72 : 0x0f71);  // phase B's rows
        barrier();
      }
    };
    epi_phase(PA, sA, 0);
    epi_phase(PB, sB, sA);
  }
}

// ------------------------------------------------------- row-halo, stride 2
//
// Stride-2 3x3 int8 convolution over 64 or 128 input channels (CS = C/64
// k-steps of 64 bytes per tap) whose padded input rows fit 64 pixels
// (Wo <= 31), 128 output channels per workgroup: the downsampling layers of
// ResNet-style networks.  The tiled kernel copies a stage's filter rows and
// patch rows into LDS for every tile and tap; here a workgroup owns
// `halo_rows` consecutive output rows (flattened n*Ho + ho) and all 128 of its
// channels, the filter stays in registers for the whole launch, and each step
// (one output row) copies only the input rows it does not share with the
// previous step: two, or three at the first row of an image.
//
// Waves 0-3 (one per SIMD) are MFMA waves.  Each holds a share of the
// 128-channel filter slice in registers (loaded straight from the packed
// filter): over 64 channels (CS = 1) wave m holds packed tiles 2(m&1),
// 2(m&1)+1 of 64-row block m>>1 (32 channels, all 9 k-steps); over 128
// channels (CS = 2) it holds all four tiles of block m>>1 and half of the 18
// k-steps, (m&1)*9 .. (m&1)*9+8 (64 channels: each patch fragment read from
// LDS feeds four MFMAs).  Each wave computes both 16-pixel tiles of the row
// (pixels past Wo read the last pixel; their results are never stored), one
// tile after the other, so that the first tile's sums go to LDS while the
// second tile's MFMAs run; its patch fragments come through a ring three
// fragments deep that runs into the next step's first fragments.  The int32
// sums go through LDS to epilogue waves 4-7: per step and per k-step half a
// 32-pixel x 128-channel int32 array, 4-channel chunk k of pixel P at
// 16 * (k ^ (P & 31)) in P's 512 bytes (conflict-free writes).  Epilogue wave
// e adds the halves (exact int32), requantises pixels 8e .. 8e+7 (16
// consecutive channels per lane, the row-halo kernel's requantisation tail)
// and stores them whole: 1 KiB contiguous per store.
//
// Input rows (1 KiB buffer->LDS copies, issued by the epilogue waves) live in
// a ring of nine 64-pixel slots.  The workgroup's rows are numbered in the
// order its steps first need them (row r of step u is number k0(u) + r, with
// k0 advancing by 2 per output row and by 3 more at each image change), and
// row number k sits in slot k % 9: the rows of three consecutive steps span
// at most nine numbers, so a copy never lands on a row still being read.
// Even pixels (X = input column + left pad) fill a slot's first 32 pixel places
// and odd pixels the rest, so a tap's 16 pixels (stride 2) are consecutive
// places, P = (X & 1) * 32 + X / 2; place P holds its 16-byte chunk c at
// P*C + 16*(c ^ ((P >> 1) & (4CS - 1))), conflict-free for 16 consecutive
// places.  Rows outside the image and columns past it read as zero
// (out-of-range offsets).  In the interval that ends with the barrier after
// MFMA step t, each epilogue wave copies its share of step t+2's new rows and
// its side tile of step t+1 (three-slot ring), requantises and stores step
// t-1, then waits for its copies (the store may stay in flight): MFMA step t+1
// reads rows that were waited for one interval earlier, and the prefetch at
// the end of MFMA step t reads only rows published before it.
constexpr int kS2Threads = 512;
constexpr int kS2Slots = 9;     // input-row slots
constexpr int kS2SideRing = 3;  // side-tile slots per epilogue wave

// Row number of row 0 of the workgroup's step for flattened output row gr
// (the workgroup starts at output row ho0 of image n0).
__device__ inline int halo_s2_k0(const ConvArgs& a, int gr, int n0, int ho0) {
  const int n = static_cast<int>(fast_div(static_cast<uint32_t>(gr), a.ho_mul, a.ho_add, a.ho_shift));
  const int ho = gr - n * a.Ho;
  if (n == n0) return 2 * (ho - ho0);
  return 2 * (a.Ho - 1 - ho0) + 3 + (n - n0 - 1) * (2 * (a.Ho - 1) + 3) + 2 * ho;
}

template <int CS, bool SIDE, bool ORDER7, bool RELU>
__global__ __launch_bounds__(kS2Threads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void conv_halo_s2_i8_kernel(ConvArgs a) {
  constexpr int CB = 64 * CS;      // bytes per input pixel
  constexpr int SLOT = 64 * CB;    // one padded input row
  constexpr int KSPLIT = CS;       // k-step parts (one sum array each)
  constexpr int NT = 2 * CS;       // 16-channel tiles per MFMA wave
  constexpr int NK = 9;            // k-steps per MFMA wave
  constexpr int NF = 2 * NK;       // fragments per step (two pixel tiles)
  constexpr int D = 3;             // patch-fragment ring depth
  constexpr int HSZ = 16384;       // one 32-pixel x 128-channel int32 array
  static_assert(NF % D == 0, "ring slots must line up across steps");
  __shared__ __attribute__((aligned(256))) char xrows[kS2Slots * SLOT];
  __shared__ __attribute__((aligned(256))) char accb[2 * KSPLIT * HSZ];
  __shared__ __attribute__((aligned(256))) char sring[SIDE ? 4 * kS2SideRing * 1024 : 16];
  __shared__ __attribute__((aligned(16))) float blds[256];
  __shared__ __attribute__((aligned(16))) float clds[256];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool mfma_role = wave < 4;
  const int g = lane >> 4;
  const int col = lane & 15;

  const int G = gridDim.x;
  const int bx = blockIdx.x;
  const int b = (G % 8 == 0) ? (bx % 8) * (G / 8) + bx / 8 : bx;
  const int rows_total = a.N * a.Ho;
  const int g0 = b * a.halo_rows;
  if (g0 >= rows_total) return;  // uniform per workgroup
  const int T = min(g0 + a.halo_rows, rows_total) - g0;  // steps (output rows)
  const int n0 = static_cast<int>(fast_div(static_cast<uint32_t>(g0), a.ho_mul, a.ho_add, a.ho_shift));
  const int ho0 = g0 - n0 * a.Ho;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.side, SIDE ? a.side_bytes : 0u);
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(a.y, a.y_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.wp, a.wp_bytes);

  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  if (mfma_role) {
    const int blk = blockIdx.y * 2 + (wave >> 1);
    const int j0 = CS == 1 ? 2 * (wave & 1) : 0;  // first packed tile of the wave
    // LDS offsets of this lane's fragments inside a row slot: tile pt, tap
    // column s, channel half c2 (the same pixels every step).
    uint32_t ad[2][3][CS];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const int wo = min(pt * 16 + col, a.Wo - 1);
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        const int X = 2 * wo + s;
        const int P = (X & 1) * 32 + (X >> 1);
#pragma unroll
        for (int c2 = 0; c2 < CS; ++c2)
          ad[pt][s][c2] =
              static_cast<uint32_t>(P * CB + 16 * ((4 * c2 + g) ^ ((P >> 1) & (4 * CS - 1))));
      }
    }
    const i32x4 zero4 = i32x4{0, 0, 0, 0};
    // The wave's k-steps kh*NK .. kh*NK + NK - 1 (kh fixed at compile time so
    // that every register index is static).
    auto run = [&](auto khc) {
      constexpr int kh = decltype(khc)::value;
      i32x4 Wf[NK][NT];
#pragma unroll
      for (int jj = 0; jj < NT; ++jj) {
        const uint32_t row = static_cast<uint32_t>(blk * 64 + (j0 + jj) * 16 + col);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          Wf[kk][jj] = __builtin_amdgcn_raw_buffer_load_b128(
              wr, row * static_cast<uint32_t>(a.wrow_bytes) + (kh * NK + kk) * 64 + g * 16, 0, 0);
      }
      // Fragment f of a step (pixel tile f / NK, k-step f % NK) from the row
      // slots rb[r] (byte offsets) of that step.
      auto frag = [&](const uint32_t (&rb)[3], int f) -> i32x4 {
        const int pt = f / NK, ks = kh * NK + f % NK;
        const int tap = ks / CS, c2 = ks % CS;
        return *reinterpret_cast<const i32x4*>(xrows + rb[tap / 3] + ad[pt][tap % 3][c2]);
      };
      auto slots = [&](int u, uint32_t (&rb)[3]) {
        const int k0 = halo_s2_k0(a, g0 + u, n0, ho0);
#pragma unroll
        for (int r = 0; r < 3; ++r)
          rb[r] = static_cast<uint32_t>(((k0 + r) % kS2Slots) * SLOT);
      };
      uint32_t rc[3], rn[3];
      slots(0, rc);
      barrier();  // steps 0 and 1's rows have landed
      i32x4 bf[D];
#pragma unroll
      for (int d = 0; d < D; ++d) bf[d] = frag(rc, d);
      for (int t = 0; t < T; ++t) {
        slots(t + 1 < T ? t + 1 : t, rn);
        char* hb = accb + ((t & 1) * KSPLIT + kh) * HSZ;
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          i32x4 acc[NT];
#pragma unroll
          for (int kk = 0; kk < NK; ++kk) {
            const int f = pt * NK + kk;
#pragma unroll
            for (int jj = 0; jj < NT; ++jj)
              acc[jj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Wf[kk][jj], bf[f % D],
                                                              kk == 0 ? zero4 : acc[jj], 0, 0, 0);
            bf[f % D] = f + D < NF ? frag(rc, f + D) : frag(rn, f + D - NF);
          }
#pragma unroll
          for (int kk = 0; kk < NK; ++kk) {
            __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
          }
          // This tile's sums: channels 64*(blk % 2) + 16g + 4(j0 + jj) + 0..3
          // of the workgroup's 128 (the first tile's writes overlap the
          // second tile's MFMAs).
          const int pix = pt * 16 + col;
#pragma unroll
          for (int jj = 0; jj < NT; ++jj) {
            const int chunk = 16 * ((wave >> 1) & 1) + 4 * g + j0 + jj;
            *reinterpret_cast<i32x4*>(hb + pix * 512 + 16 * (chunk ^ (pix & 31))) = acc[jj];
          }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): hand-off written
        barrier();
#pragma unroll
        for (int r = 0; r < 3; ++r) rc[r] = rn[r];
      }
      barrier();  // the epilogue waves' last step
    };
    if constexpr (CS == 2) {
      if (wave & 1)
        run(std::integral_constant<int, 1>{});
      else
        run(std::integral_constant<int, 0>{});
    } else {
      run(std::integral_constant<int, 0>{});
    }
  } else {
    const int e = wave - 4;
    const __amdgpu_buffer_rsrc_t br = make_rsrc(a.bias, static_cast<uint32_t>(a.K) * 4u);
    const __amdgpu_buffer_rsrc_t cr =
        make_rsrc(a.cis_vec, a.cis_vec ? static_cast<uint32_t>(a.K) * 4u : 0u);
    // This wave copies KiB e + 4c (c < CS) of every row: the source offset
    // inside the row, per lane (out-of-range columns get 2^31, which keeps
    // the sum with any row's offset, below 2^31, out of range).
    // (A fixed bound: with a bound that depends on CS, captured by the lambda
    // below, clang's host pass drops the kernel's launch stub.)
    uint32_t lane_off[2];
#pragma unroll
    for (int c = 0; c < CS; ++c) {
      const int pos = (e + 4 * c) * 1024 + lane * 16;
      const int P = pos / CB;
      const int X = P < 32 ? 2 * P : 2 * (P - 32) + 1;
      const int ch = ((pos % CB) >> 4) ^ ((P >> 1) & (4 * CS - 1));
      const int wi = X - a.pl;
      lane_off[c] = static_cast<unsigned>(wi) < static_cast<unsigned>(a.W)
                        ? static_cast<uint32_t>(wi * CB + ch * 16)
                        : kOutOfRange;
    }
    // This wave's share of step u's new rows (all three at the first step and
    // at the first row of an image, else rows 1 and 2).
    auto copy_rows = [&](int u) {
      if (u >= T) return;
      const int gr = g0 + u;
      const int n = static_cast<int>(fast_div(static_cast<uint32_t>(gr), a.ho_mul, a.ho_add, a.ho_shift));
      const int ho = gr - n * a.Ho;
      const int k0 = halo_s2_k0(a, gr, n0, ho0);
      for (int r = (u == 0 || ho == 0) ? 0 : 1; r < 3; ++r) {
        const int hi = 2 * ho - a.pt + r;
        const bool row_ok = static_cast<unsigned>(hi) < static_cast<unsigned>(a.H);
        const uint32_t rbase = static_cast<uint32_t>((n * a.H + hi) * a.W * CB);
        char* slot = xrows + ((k0 + r) % kS2Slots) * SLOT;
#pragma unroll
        for (int c = 0; c < CS; ++c)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(slot + (e + 4 * c) * 1024), 16,
                                                   row_ok ? rbase + lane_off[c] : kOutOfRange, 0,
                                                   0, 0);
      }
    };
    // Side tile of this wave's 8 pixels at step u into ring slot u % 3.
    auto copy_side = [&](int u) {
      const int px = 8 * e + (lane >> 3);
      const bool ok = u < T && px < a.Wo;
      const uint32_t src = ok ? static_cast<uint32_t>(((g0 + u) * a.Wo + px) * a.K +
                                                      blockIdx.y * 128 + (lane & 7) * 16)
                              : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          sr, (lds_ptr_t)(sring + (e * kS2SideRing + u % kS2SideRing) * 1024), 16, src, 0, 0, 0);
    };
    copy_rows(0);
    copy_rows(1);
    if (e < 2) {
      const uint32_t off = lane < 32 ? static_cast<uint32_t>((blockIdx.y * 128 + 4 * lane) * 4)
                                     : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(e == 0 ? br : cr, (lds_ptr_t)(e == 0 ? blds : clds),
                                               16, off, 0, 0, 0);
    }
    if constexpr (SIDE) copy_side(0);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): steps 0 and 1 are read during step 0
    barrier();
    const int px = lane >> 3, qq = lane & 7;
    const int pix = 8 * e + px;
    const int ch = blockIdx.y * 128 + 16 * qq;
    float bias[16], cis_v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      bias[i] = blds[16 * qq + i];
      cis_v[i] = a.cis_vec ? clds[16 * qq + i] : a.cis;
    }
    const float sis = a.sis;
    const float lo_b = kRoundMagic + (a.relu ? 0.0f : -128.0f), hi_b = kRoundMagic + 127.0f;
    for (int t = 0; t <= T; ++t) {
      copy_rows(t + 2);
      if constexpr (SIDE) copy_side(t + 1);
      if (t >= 1) {
        const int q = t - 1;
        i32x4 acc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int off = pix * 512 + 16 * ((4 * qq + i) ^ (pix & 31));
          acc[i] = *reinterpret_cast<const i32x4*>(accb + (q & 1) * KSPLIT * HSZ + off);
          if constexpr (KSPLIT == 2)
            acc[i] += *reinterpret_cast<const i32x4*>(accb + ((q & 1) * KSPLIT + 1) * HSZ + off);
        }
        i32x4 sd = i32x4{0, 0, 0, 0};
        if constexpr (SIDE) {
          // Landed before the barrier that ended the previous interval; read
          // in an asm block so that the compiler adds no wait for the copies
          // in flight into the ring's other slots.
          const uint32_t side_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
              (lds_ptr_t)(sring + (e * kS2SideRing + q % kS2SideRing) * 1024 + lane * 16)));
          asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                       : "=&v"(sd)
                       : "v"(side_addr)
                       : "memory");
        }
        float tv[16];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float f = static_cast<float>(acc[i][j]);
            tv[4 * i + j] = ORDER7 ? __builtin_fmaf(f, cis_v[4 * i + j], bias[4 * i + j])
                                   : f * cis_v[4 * i + j];
          }
        uint32_t w[4];
        halo_epilogue_tail<SIDE, ORDER7, RELU>(tv, sd, bias, sis, lo_b, hi_b, w);
        const bool ok = pix < a.Wo;
        const uint32_t off = ok ? static_cast<uint32_t>(((g0 + q) * a.Wo + pix) * a.K + ch)
                                : kOutOfRange;
        store_words<16>(w, yr, off);
        // This interval's copies have landed (the store may stay in flight).
        __builtin_amdgcn_s_waitcnt(0x0f71);  // vmcnt(1)
      } else {
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
      }
      barrier();
    }
  }
}

// ------------------------------------------------- full-size VALID as a GEMM
//
// A filter as large as the image with VALID padding has a single output
// pixel per image, and the convolution is one matrix product (TensorFlow
// conv_ops_fused_int8.cc, LaunchFusedConv2DOpCpuInt8Helper, the second GEMM
// special case):  y[n][k] = sum_j x[n][j] * w[j][k],  j = (r, s, c) over the
// whole image, x viewed as [N][H*W*C] and the filter as [R*S*C][K].  Both
// operands are contiguous along j (an NHWC image; a packed filter row).
//
// The product is thin (N images) and deep (H*W*C), and the filter is almost
// all of its bytes: the work is streaming the filter.  To put every CU on
// it, the reduction is split into ranges: a workgroup owns 32 output
// channels, 32 images and one range (grid: channel tiles x ranges x image
// tiles).  Its 16 waves each stream a contiguous part of the range with
// fragments loaded straight from global memory into registers (x, re-read
// by every channel tile, stays in L2), four k-steps of loads in flight, and
// add their 32 x 32 partial sums through LDS in wave order.  The workgroup
// writes its partial tile [range][n][k] (int32 for int8, fp32 otherwise) to
// the workspace.  A second kernel adds the ranges in range order and runs
// the fused epilogue, so every run gives the same bits.  (Adding the ranges
// in the last workgroup of each tile instead needs a device-scope release
// per workgroup, an L2 write-back each: measured 10x slower.)  Requires
// R*S*C*esize to be whole 64-byte k-steps.
constexpr int kGemmWaves = 16;
constexpr int kGemmThreads = 64 * kGemmWaves;
constexpr int kGemmBN = 32;    // output channels per workgroup (half a packed 64-row block)
constexpr int kGemmBatch = 4;  // k-steps of loads in flight per wave

template <int DT>
__global__ __launch_bounds__(kGemmThreads) void conv_gemm_splitk_kernel(ConvArgs a) {
  using Acc = typename Dt<DT>::Acc;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int g = lane >> 4, col = lane & 15;
  const int ct = blockIdx.x, split = blockIdx.y, nt = blockIdx.z, n0 = nt * 32;
  const int row_bytes = a.Kg * (16 / Dt<DT>::kChunk);  // bytes of one image / filter row
  const int nks = row_bytes >> 6;                      // 64-byte k-steps
  // This workgroup's k-steps [kb, ke), and this wave's contiguous part.
  const int kb = split * a.gemm_kps;
  const int ke = min(kb + a.gemm_kps, nks);
  const int per_wave = (a.gemm_kps + kGemmWaves - 1) / kGemmWaves;
  const int wb = kb + wave * per_wave;
  const int we = min(wb + per_wave, ke);
  // Packed rows 32ct + 16jj + col (jj = 0, 1) hold, for lane group g, the
  // channels chb(g) + 4jj .. +3 with chb(g) = 64(ct/2) + 16g + 8(ct%2): eight
  // consecutive channels per lane (the repack's order inside a 64-row block).
  const int chb = 64 * (ct >> 1) + 8 * (ct & 1);

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.wp, a.wp_bytes);
  uint32_t xo[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int n = n0 + 16 * i + col;
    xo[i] = n < a.N ? static_cast<uint32_t>(n * row_bytes + 16 * g) : kOutOfRange;
  }
  const uint32_t wo = static_cast<uint32_t>((kGemmBN * ct + col) * a.wrow_bytes + 16 * g);

  Acc acc[2][2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[jj][i] = Acc{0, 0, 0, 0};
  for (int k0 = wb; k0 < we; k0 += kGemmBatch) {
    i32x4 fa[kGemmBatch][2], fb[kGemmBatch][2];
#pragma unroll
    for (int b = 0; b < kGemmBatch; ++b) {
      const bool live = k0 + b < we;
      const uint32_t kbyte = static_cast<uint32_t>((k0 + b) * 64);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        fa[b][jj] = __builtin_amdgcn_raw_buffer_load_b128(
            wr, live ? wo + static_cast<uint32_t>(16 * jj * a.wrow_bytes) + kbyte : kOutOfRange,
            0, 0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fb[b][i] = __builtin_amdgcn_raw_buffer_load_b128(
            xr, live && xo[i] != kOutOfRange ? xo[i] + kbyte : kOutOfRange, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < kGemmBatch; ++b)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          acc[jj][i] = mma_chunk(fa[b][jj], fb[b][i], acc[jj][i], static_cast<Dt<DT>*>(nullptr));
  }

  // The waves' tiles, added through LDS in wave order: slot q = 2jj + i of
  // wave w holds lane l's four values at ((w * 4 + q) * 64 + l) * 16.
  __shared__ __attribute__((aligned(16))) char red[kGemmWaves * 4 * 1024];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<Acc*>(red + ((wave * 4 + 2 * jj + i) * 64 + lane) * 16) = acc[jj][i];
  __syncthreads();
  const int t = threadIdx.x;
  const int64_t tile_stride = static_cast<int64_t>(a.N) * a.Kp * 4;  // bytes of one range's tiles
  char* part = static_cast<char*>(a.part);
  if (t < 256) {
    // Thread t: slot q = t / 64 of lane l = t % 64, i.e. channels
    // chb(l / 16) + 4jj .. +3 of image n0 + 16i + l % 16.
    const int q = t >> 6, l = t & 63;
    Acc sum = *reinterpret_cast<const Acc*>(red + (q * 64 + l) * 16);
#pragma unroll
    for (int w = 1; w < kGemmWaves; ++w)
      sum = sum + *reinterpret_cast<const Acc*>(red + ((w * 4 + q) * 64 + l) * 16);
    const int n = n0 + 16 * (q & 1) + (l & 15);
    const int ch = chb + 16 * (l >> 4) + 4 * (q >> 1);
    if (n < a.N)
      *reinterpret_cast<Acc*>(part + split * tile_stride + (static_cast<int64_t>(n) * a.Kp + ch) * 4) =
          sum;
  }
}

// Sum of the ranges (in range order) and the fused epilogue: thread =
// 8 consecutive channels of one image; workgroups of one wave, so the sum's
// reads spread over many CUs.  The partial tiles are read eight ranges at a
// time (all eight loads in flight), then added in range order.
constexpr int kGemmReduceThreads = 64;

template <int DT, bool KVEC>
__global__ __launch_bounds__(kGemmReduceThreads) void conv_gemm_reduce_kernel(ConvArgs a) {
  using Acc = typename Dt<DT>::Acc;
  using Elem = typename std::conditional<DT == FCONV_INT8, int32_t, float>::type;
  const int groups = a.Kp >> 3;
  const int id = blockIdx.x * kGemmReduceThreads + threadIdx.x;
  if (id >= a.N * groups) return;
  const int n = id / groups, ch0 = (id - n * groups) * 8;
  if (ch0 >= a.K) return;
  const int64_t tile_stride = static_cast<int64_t>(a.N) * a.Kp * 4;  // bytes of one range's tiles
  const char* src = static_cast<const char*>(a.part) + (static_cast<int64_t>(n) * a.Kp + ch0) * 4;
  // The epilogue's per-channel values and side chunk first: their loads do
  // not depend on the sums, so they are in flight with the partial tiles'.
  i32x4 sc = i32x4{0, 0, 0, 0};
  float bias[8], cis[8];
  FloatEpiParams<8> P;
  if constexpr (DT == FCONV_INT8) {
    if (a.use_side) sc = load_side_chunk<8>(a, n, ch0, KVEC);
    load_bias<8>(a, ch0, KVEC, bias);
    load_scales<8>(a, ch0, KVEC, cis);
  } else {
    P.load(a, ch0, KVEC);
  }
  Acc s0 = Acc{0, 0, 0, 0}, s1 = Acc{0, 0, 0, 0};
  for (int sp0 = 0; sp0 < a.gemm_splits; sp0 += 8) {
    Acc v0[8], v1[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (sp0 + u < a.gemm_splits) {
        const char* q = src + (sp0 + u) * tile_stride;
        v0[u] = *reinterpret_cast<const Acc*>(q);
        v1[u] = *reinterpret_cast<const Acc*>(q + 16);
      } else {
        v0[u] = v1[u] = Acc{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      s0 = s0 + v0[u];
      s1 = s1 + v1[u];
    }
  }
  Elem v[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = s0[e];
    v[4 + e] = s1[e];
  }
  if constexpr (DT == FCONV_INT8)
    epilogue_store_i8<8>(v, a, n, ch0, KVEC, sc, bias, cis);
  else
    epilogue_store_float<DT, 8>(v, a, n, ch0, KVEC, P);
}

// ------------------------------------------------------------- dispatch

template <int DT>
hipError_t launch_pack(const fconv_plan_s* p, const void* w, void* wp, hipStream_t s) {
  const int64_t chunks = static_cast<int64_t>(p->Kp) * (p->KgP / p->chunk_elems + 1);
  const int blocks = static_cast<int>((chunks + 255) / 256);
  hipLaunchKernelGGL(pack_filter_kernel<DT>, dim3(blocks), dim3(256), 0, s, w, wp, p->d.K,
                     p->Kg, p->KgP, p->Kp);
  return hipGetLastError();
}

template <int DT, int MODE>
hipError_t launch_general_mode(const fconv_plan_s* p, const ConvArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((p->M + kTileM - 1) / kTileM),
                  static_cast<unsigned>(p->Kp / kTileN));
  if (p->d.K % 16 == 0)
    hipLaunchKernelGGL((conv_general_kernel<DT, MODE, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((conv_general_kernel<DT, MODE, false>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_general(const fconv_plan_s* p, const ConvArgs& a, hipStream_t s) {
  switch (p->load_mode) {
    case kLoadTap: return launch_general_mode<DT, kLoadTap>(p, a, s);
    case kLoadChunk: return launch_general_mode<DT, kLoadChunk>(p, a, s);
    default: return launch_general_mode<DT, kLoadElem>(p, a, s);
  }
}

template <int DT, int PT, int D>
hipError_t launch_rf_pt(const fconv_plan_s* p, const ConvArgs& a, hipStream_t s) {
  const size_t lds = static_cast<size_t>(kRfBN) * a.wrow_bytes;
  const auto kern = conv_rf_kernel<DT, PT, D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>((p->M + 64 * PT - 1) / (64 * PT)),
                  static_cast<unsigned>(p->Kp / kRfBN));
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_rf(const fconv_plan_s* p, const ConvArgs& a, hipStream_t s) {
  const int key = p->pixel_tiles * 100 + p->ring_depth;
  switch (key) {
    case 104: return launch_rf_pt<DT, 1, 4>(p, a, s);
    case 109: return launch_rf_pt<DT, 1, 9>(p, a, s);
    case 204: return launch_rf_pt<DT, 2, 4>(p, a, s);
    case 209: return launch_rf_pt<DT, 2, 9>(p, a, s);
    case 402: return launch_rf_pt<DT, 4, 2>(p, a, s);
    case 404: return launch_rf_pt<DT, 4, 4>(p, a, s);
    default: return launch_rf_pt<DT, 2, 4>(p, a, s);
  }
}

// Compute units of the current device, queried once per device.  Runs on
// several host threads at once are allowed, so the cache entries are atomics:
// two threads may both query a device the first time and store the same value.
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int R, int S, int CS>
hipError_t launch_stream_shape(const fconv_plan_s* p, const ConvArgs& a, hipStream_t s) {
  const int cus = device_cu_count();
  int grid = (a.tiles + 3) / 4;  // at least one tile per wave
  if (grid > cus) grid = cus;
  const dim3 g(static_cast<unsigned>(grid), static_cast<unsigned>(p->Kp / 64));
  const size_t lds = static_cast<size_t>(64) * a.wrow_bytes;
  if (a.use_side && a.cudnn7)
    hipLaunchKernelGGL((conv_stream_i8_kernel<R, S, CS, true, 1, true>), g, dim3(kThreads), lds, s, a);
  else if (a.use_side)
    hipLaunchKernelGGL((conv_stream_i8_kernel<R, S, CS, true, 1, false>), g, dim3(kThreads), lds, s, a);
  else if (a.cudnn7)
    hipLaunchKernelGGL((conv_stream_i8_kernel<R, S, CS, false, 1, true>), g, dim3(kThreads), lds, s, a);
  else
    hipLaunchKernelGGL((conv_stream_i8_kernel<R, S, CS, false, 1, false>), g, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_stream(const fconv_plan_s* p, const ConvArgs& a, hipStream_t s) {
  const int cs = p->d.C / 64;
  if (p->d.R == 3 && p->d.S == 3 && cs == 1) return launch_stream_shape<3, 3, 1>(p, a, s);
  if (p->d.R == 1 && p->d.S == 1) {
    switch (cs) {
      case 1: return launch_stream_shape<1, 1, 1>(p, a, s);
      case 2: return launch_stream_shape<1, 1, 2>(p, a, s);
      case 4: return launch_stream_shape<1, 1, 4>(p, a, s);
      case 8: return launch_stream_shape<1, 1, 8>(p, a, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

// Whether both phases of the row-halo kernel fit their LDS arrays when each
// workgroup takes `rows` output rows (phase A two rows, phase B the rest):
// input-row slots (rows + (R-1) per image the phase touches), checked exactly
// for every workgroup.
bool halo_fits(const fconv_plan_s* p, int rows) {
  const int64_t rows_total = static_cast<int64_t>(p->d.N) * p->Ho;
  const int slots[2] = {kHaloSlotsA, kHaloSlotsB};
  const int len[2] = {std::min(kHaloRowsA, rows), rows - std::min(kHaloRowsA, rows)};
  for (int64_t g0 = 0; g0 < rows_total; g0 += rows) {
    int64_t p0 = g0;
    for (int ph = 0; ph < 2; ++ph) {
      const int64_t p1 = std::min<int64_t>(p0 + len[ph], rows_total);
      if (p1 > p0) {
        const int64_t images = (p1 - 1) / p->Ho - p0 / p->Ho + 1;
        if ((p1 - p0) + (p->d.R - 1) * images > slots[ph]) return false;
      }
      p0 = std::max(p0, p1);
    }
  }
  return true;
}

template <int R, int S, bool SIDE, bool ORDER7>
void launch_halo_relu(dim3 g, const ConvArgs& a, hipStream_t s) {
  if (a.relu)
    hipLaunchKernelGGL((conv_halo_i8_kernel<R, S, SIDE, ORDER7, true>), g, dim3(kHaloThreads), 0,
                       s, a);
  else
    hipLaunchKernelGGL((conv_halo_i8_kernel<R, S, SIDE, ORDER7, false>), g, dim3(kHaloThreads), 0,
                       s, a);
}

template <int R, int S>
hipError_t launch_halo_kernel(dim3 g, const ConvArgs& a, hipStream_t s) {
  if (a.use_side && a.cudnn7)
    launch_halo_relu<R, S, true, true>(g, a, s);
  else if (a.use_side)
    launch_halo_relu<R, S, true, false>(g, a, s);
  else if (a.cudnn7)
    launch_halo_relu<R, S, false, true>(g, a, s);
  else
    launch_halo_relu<R, S, false, false>(g, a, s);
  return hipGetLastError();
}

template <int R, int S>
hipError_t launch_halo_shape(const fconv_plan_s* p, const ConvArgs& a0, hipStream_t s) {
  ConvArgs a = a0;
  const int cus = device_cu_count();
  const int rows_total = p->d.N * p->Ho;
  int rows = p->halo_rows > 0 ? std::min(p->halo_rows, rows_total)
                              : (rows_total + cus - 1) / cus;
  while (rows > 1 && !halo_fits(p, rows)) --rows;
  if (!halo_fits(p, rows)) return hipErrorInvalidValue;
  a.halo_rows = rows;
  a.halo_rows_a = std::min(kHaloRowsA, rows);
  const dim3 g(static_cast<unsigned>((rows_total + rows - 1) / rows), static_cast<unsigned>(p->Kp / 64));
  return launch_halo_kernel<R, S>(g, a, s);
}

hipError_t launch_halo(const fconv_plan_s* p, const ConvArgs& a, hipStream_t s) {
  if (p->d.R == 3 && p->d.S == 3) return launch_halo_shape<3, 3>(p, a, s);
  return hipErrorInvalidValue;
}

template <int CS, bool SIDE, bool ORDER7>
void launch_halo_s2_relu(dim3 g, const ConvArgs& a, hipStream_t s) {
  if (a.relu)
    hipLaunchKernelGGL((conv_halo_s2_i8_kernel<CS, SIDE, ORDER7, true>), g, dim3(kS2Threads), 0,
                       s, a);
  else
    hipLaunchKernelGGL((conv_halo_s2_i8_kernel<CS, SIDE, ORDER7, false>), g, dim3(kS2Threads), 0,
                       s, a);
}

template <int CS>
void launch_halo_s2_cs(dim3 g, const ConvArgs& a, hipStream_t s) {
  if (a.use_side && a.cudnn7)
    launch_halo_s2_relu<CS, true, true>(g, a, s);
  else if (a.use_side)
    launch_halo_s2_relu<CS, true, false>(g, a, s);
  else if (a.cudnn7)
    launch_halo_s2_relu<CS, false, true>(g, a, s);
  else
    launch_halo_s2_relu<CS, false, false>(g, a, s);
}

// The stride-2 row kernel: `halo_rows` output rows per workgroup (by default
// the rows spread evenly over the CUs), 128 output channels per workgroup.
hipError_t launch_halo_s2(const fconv_plan_s* p, const ConvArgs& a0, hipStream_t s) {
  const fconv_desc& d = p->d;
  if (!(d.R == 3 && d.S == 3 && d.stride_h == 2 && d.stride_w == 2 &&
        (d.C == 64 || d.C == 128) && d.K % 128 == 0 && p->Wo <= 31))
    return hipErrorInvalidValue;
  ConvArgs a = a0;
  const int cus = device_cu_count();
  const int rows_total = d.N * p->Ho;
  const int rows = p->halo_rows > 0 ? std::min(p->halo_rows, rows_total)
                                    : (rows_total + cus - 1) / cus;
  a.halo_rows = rows;
  a.halo_rows_a = rows;
  const dim3 g(static_cast<unsigned>((rows_total + rows - 1) / rows),
               static_cast<unsigned>(d.K / 128));
  if (d.C == 64)
    launch_halo_s2_cs<1>(g, a, s);
  else
    launch_halo_s2_cs<2>(g, a, s);
  return hipGetLastError();
}

hipError_t launch_pack_any(const fconv_plan_s* p, const void* w, void* wp, hipStream_t s) {
  switch (p->d.dtype) {
    case FCONV_INT8: return launch_pack<FCONV_INT8>(p, w, wp, s);
    case FCONV_BF16: return launch_pack<FCONV_BF16>(p, w, wp, s);
    default: return launch_pack<FCONV_FP32>(p, w, wp, s);
  }
}

template <int DT>
hipError_t launch_tile(const fconv_plan_s* p, const ConvArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((p->M + kTileBM - 1) / kTileBM),
                  static_cast<unsigned>((p->Kp + kTileBN - 1) / kTileBN));
  // Two stages per barrier where measured faster or equal: the layers with
  // one 128-channel tile (K <= 128: 4% on the CBNA 5x5 and 7x7 layers, equal
  // on the strided int8 layer); one per stage otherwise (3% slower with two
  // on the 256-channel bf16 layer).
  // 64-pixel tiles where 128-pixel ones would leave at least half the CUs
  // idle (the CBNA layers: 98 tiles), unless the plan pins the height.
  // 256-pixel tiles where 128-pixel ones would need a second round over the
  // CUs and 256-pixel ones fit in one (the strided int8 layer: 392 -> 196).
  const int64_t tiles = static_cast<int64_t>(grid.x) * grid.y;
  const int64_t cus = device_cu_count();
  const int64_t tall_tiles = (p->M + kTall - 1) / kTall * grid.y;
  const bool tall = p->pixel_tiles == 4 || (p->pixel_tiles == 0 && tiles > cus && tall_tiles <= cus);
  const bool bm64 = p->pixel_tiles == 1 || (p->pixel_tiles == 0 && tiles * 2 <= cus);
  // 64- and 128-pixel tiles of int8 and bf16: copy waves beside the MFMA
  // waves, unless FCONV_TILE_ROLES=0.
  if constexpr (DT != FCONV_FP32) {
    if (p->tile_roles && !tall) {
      if (bm64) {
        const dim3 grid64(static_cast<unsigned>((p->M + 63) / 64), grid.y);
        hipLaunchKernelGGL((conv_tile_cw_kernel<DT, true, 64>), grid64, dim3(kCwThreads), 0, s, a);
      } else {
        hipLaunchKernelGGL((conv_tile_cw_kernel<DT, true, 128>), grid, dim3(kCwThreads), 0, s, a);
      }
      return hipGetLastError();
    }
  }
  if (tall) {
    const dim3 grid256(static_cast<unsigned>((p->M + kTall - 1) / kTall), grid.y);
    hipLaunchKernelGGL((conv_tile256_kernel<DT, true>), grid256, dim3(kTileThreads), 0, s, a);
  } else if (bm64) {
    const dim3 grid64(static_cast<unsigned>((p->M + 63) / 64), grid.y);
    if (p->d.K <= kTileBN)
      hipLaunchKernelGGL((conv_tile_kernel<DT, true, true, 64>), grid64, dim3(kTileThreads), 0, s, a);
    else
      hipLaunchKernelGGL((conv_tile_kernel<DT, true, false, 64>), grid64, dim3(kTileThreads), 0, s, a);
  } else if (p->d.K <= kTileBN) {
    hipLaunchKernelGGL((conv_tile_kernel<DT, true, true, 128>), grid, dim3(kTileThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((conv_tile_kernel<DT, true, false, 128>), grid, dim3(kTileThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_gemm(const fconv_plan_s* p, const ConvArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p->Kp / kGemmBN), static_cast<unsigned>(p->gemm_splits),
                  static_cast<unsigned>((p->d.N + 31) / 32));
  hipLaunchKernelGGL(conv_gemm_splitk_kernel<DT>, grid, dim3(kGemmThreads), 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = static_cast<int64_t>(p->d.N) * (p->Kp / 8);
  const dim3 g2(static_cast<unsigned>((threads + kGemmReduceThreads - 1) / kGemmReduceThreads));
  if (p->d.K % 8 == 0)
    hipLaunchKernelGGL((conv_gemm_reduce_kernel<DT, true>), g2, dim3(kGemmReduceThreads), 0, s, a);
  else
    hipLaunchKernelGGL((conv_gemm_reduce_kernel<DT, false>), g2, dim3(kGemmReduceThreads), 0, s,
                       a);
  return hipGetLastError();
}

hipError_t launch_conv(const fconv_plan_s* p, const ConvArgs& a, hipStream_t s) {
  if (p->variant == kGemm) {
    switch (p->d.dtype) {
      case FCONV_INT8: return launch_gemm<FCONV_INT8>(p, a, s);
      case FCONV_BF16: return launch_gemm<FCONV_BF16>(p, a, s);
      default: return launch_gemm<FCONV_FP32>(p, a, s);
    }
  }
  if (p->variant == kStream) return launch_stream(p, a, s);
  if (p->variant == kHalo) return launch_halo(p, a, s);
  if (p->variant == kHaloS2) return launch_halo_s2(p, a, s);
  if (p->variant == kTiled) {
    switch (p->d.dtype) {
      case FCONV_INT8: return launch_tile<FCONV_INT8>(p, a, s);
      case FCONV_BF16: return launch_tile<FCONV_BF16>(p, a, s);
      default: return launch_tile<FCONV_FP32>(p, a, s);
    }
  }
  if (p->variant == kResidentFilter) {
    switch (p->d.dtype) {
      case FCONV_INT8: return launch_rf<FCONV_INT8>(p, a, s);
      case FCONV_BF16: return launch_rf<FCONV_BF16>(p, a, s);
      default: return launch_rf<FCONV_FP32>(p, a, s);
    }
  }
  switch (p->d.dtype) {
    case FCONV_INT8: return launch_general<FCONV_INT8>(p, a, s);
    case FCONV_BF16: return launch_general<FCONV_BF16>(p, a, s);
    default: return launch_general<FCONV_FP32>(p, a, s);
  }
}

}  // namespace
}  // namespace fconv

namespace fconv {
namespace {

// Kernel arguments of one run of the plan.
ConvArgs make_conv_args(const fconv_plan_s* p, const fconv_args* args) {
  ConvArgs a;
  a.x = args->x;
  a.wp = args->workspace;
  a.bias = args->bias;
  a.side = static_cast<const int8_t*>(args->side);
  a.bn_gamma = args->bn_gamma;
  a.bn_beta = args->bn_beta;
  a.bn_mean = args->bn_mean;
  a.bn_var = args->bn_var;
  a.y = args->y;
  a.cis = args->conv_input_scale;
  a.cis_vec = args->conv_input_scales;
  a.cudnn7 = p->cudnn7;
  a.sis = args->side_input_scale;
  a.bn_eps = args->bn_eps;
  a.N = p->d.N; a.H = p->d.H; a.W = p->d.W; a.C = p->d.C; a.K = p->d.K;
  a.R = p->d.R; a.S = p->d.S; a.sh = p->d.stride_h; a.sw = p->d.stride_w;
  a.pt = p->pt; a.pl = p->pl; a.Ho = p->Ho; a.Wo = p->Wo;
  a.M = static_cast<int32_t>(p->M);
  a.Kg = p->Kg;
  a.KgP = p->KgP;
  a.wrow_bytes = p->wrow_bytes;
  a.x_bytes = static_cast<uint32_t>(p->x_elems * p->esize);
  a.y_bytes = static_cast<uint32_t>(p->y_elems * p->esize);
  a.side_bytes = static_cast<uint32_t>(p->y_elems);
  a.wp_bytes = static_cast<uint32_t>(p->pack_bytes);
  a.part = p->part_offset ? static_cast<char*>(args->workspace) + p->part_offset : nullptr;
  a.gemm_splits = p->gemm_splits;
  a.gemm_kps = p->gemm_kps;
  a.Kp = p->Kp;
  a.tiles = static_cast<int32_t>((p->M + 15) / 16);
  a.wo_mul = p->wo_div.mul; a.wo_add = p->wo_div.add; a.wo_shift = p->wo_div.shift;
  a.ho_mul = p->ho_div.mul; a.ho_add = p->ho_div.add; a.ho_shift = p->ho_div.shift;
  // TensorFlow's output kernel skips the side input when its scale is zero.
  a.use_side = p->op_side && args->side_input_scale != 0.0f;
  a.use_bias = p->op_bias;
  a.use_bn = p->op_bn;
  a.relu = p->op_relu;
  a.act = p->act;
  a.act_alpha = args->activ_alpha;
  a.act_beta = args->activ_beta;
  return a;
}

// Normwise difference of two outputs of the plan, max|a - b| / max|a|
// (int8: 0 if bit-identical, else 1).
double output_difference(const fconv_plan_s* p, const std::vector<uint8_t>& a,
                         const std::vector<uint8_t>& b) {
  if (p->d.dtype == FCONV_INT8) return memcmp(a.data(), b.data(), a.size()) == 0 ? 0.0 : 1.0;
  double num = 0.0, den = 0.0;
  const size_t n = static_cast<size_t>(p->y_elems);
  for (size_t i = 0; i < n; ++i) {
    float x, y;
    if (p->d.dtype == FCONV_BF16) {
      uint32_t ux = static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(a.data())[i]) << 16;
      uint32_t uy = static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(b.data())[i]) << 16;
      memcpy(&x, &ux, 4);
      memcpy(&y, &uy, 4);
    } else {
      x = reinterpret_cast<const float*>(a.data())[i];
      y = reinterpret_cast<const float*>(b.data())[i];
    }
    num = std::max(num, static_cast<double>(std::fabs(x - y)));
    den = std::max(den, static_cast<double>(std::fabs(x)));
  }
  return den > 0.0 ? num / den : num;
}

}  // namespace
}  // namespace fconv

// ---------------------------------------------- runs that allocate nothing
//
// fconv_plan_run_no_alloc keeps the run's scratch (the repacked filter) in
// this file-scope device array instead of a caller workspace.  Each device
// holds its own copy at its own address until the process ends; host code
// reaches it only through the per-device address hipGetSymbolAddress
// returns (the array's name is a host-side stand-in, not a device address).
constexpr size_t kNoAllocScratchBytes = FCONV_NO_ALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace fconv {
namespace {

// Device address of `scratch` on device `dev`, looked up once per device with
// that device current; nullptr if the runtime reports an error.
void* scratch_address(int dev) {
  static std::mutex mu;
  static void* addr[64] = {};
  if (dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev]) return addr[dev];
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || !ptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  addr[dev] = ptr;
  return ptr;
}

}  // namespace
}  // namespace fconv

extern "C" {

fconv_status fconv_plan_pack_filter(fconv_plan p, void* stream, const void* w,
                                    void* workspace, size_t workspace_bytes) {
  fconv_status st = fconv::check_pack_args(p, w, workspace, workspace_bytes);
  if (st != FCONV_OK) return st;
  hipError_t e = fconv::launch_pack_any(p, w, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FCONV_OK : FCONV_ERR_DEVICE;
}

fconv_status fconv_plan_run(fconv_plan p, void* stream, const fconv_args* args) {
  fconv_status st = fconv::check_run_args(p, args);
  if (st != FCONV_OK) return st;
  if (p->M == 0) return FCONV_OK;  // empty batch: nothing to compute
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!(args->flags & FCONV_RUN_FILTER_PREPACKED)) {
    if (fconv::launch_pack_any(p, args->w, args->workspace, s) != hipSuccess)
      return FCONV_ERR_DEVICE;
  }
  fconv::ConvArgs a = fconv::make_conv_args(p, args);
  if (fconv::launch_conv(p, a, s) != hipSuccess) return FCONV_ERR_DEVICE;
  return FCONV_OK;
}


fconv_status fconv_plan_run_no_alloc(fconv_plan p, void* stream, const fconv_args* args) {
  if (!p || !args) return FCONV_ERR_INVALID_ARG;
  if (p->ws_bytes > kNoAllocScratchBytes) return FCONV_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = -1;
  if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) {
    (void)hipGetLastError();
    return FCONV_ERR_DEVICE;
  }
  void* ws = fconv::scratch_address(dev);
  if (!ws) return FCONV_ERR_DEVICE;
  fconv_args a = *args;
  a.workspace = ws;
  a.workspace_bytes = kNoAllocScratchBytes;
  return fconv_plan_run(p, stream, &a);
}

fconv_status fconv_plan_autotune(fconv_plan p, void* stream, const fconv_args* args,
                                 int32_t repeats, float* best_us) {
  fconv_status st = fconv::check_run_args(p, args);
  if (st != FCONV_OK) return st;
  if (repeats < 1 || repeats > 100000) return FCONV_ERR_INVALID_ARG;
  if (p->M == 0) return FCONV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!(args->flags & FCONV_RUN_FILTER_PREPACKED) &&
      fconv::launch_pack_any(p, args->w, args->workspace, s) != hipSuccess)
    return FCONV_ERR_DEVICE;
  const fconv::ConvArgs a = fconv::make_conv_args(p, args);
  fconv::KernelConfig cand[16];
  const int n = fconv::list_configs(p, cand, 16);
  const size_t ybytes = static_cast<size_t>(p->y_elems) * p->esize;
  std::vector<uint8_t> ref(ybytes), out(ybytes);
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return FCONV_ERR_DEVICE;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return FCONV_ERR_DEVICE;
  }
  // Agreement with the plan's own configuration (the first candidate):
  // bit-exact for int8.  Float configurations differ only in the order of
  // their fp32 sums: for bf16 output that flips at most an ulp or two of the
  // rounded result (2^-8 relative each), so 8e-3 normwise; fp32 1e-5.
  const double tol = p->d.dtype == FCONV_INT8 ? 0.0 : p->d.dtype == FCONV_BF16 ? 8e-3 : 1e-5;
  float best = -1.0f;
  int best_i = 0;
  st = FCONV_OK;
  for (int i = 0; i < n && st == FCONV_OK; ++i) {
    fconv_plan_s q = *p;
    fconv::apply_config(&q, cand[i]);
    if (fconv::launch_conv(&q, a, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess) {
      if (i == 0) st = FCONV_ERR_DEVICE;
      (void)hipGetLastError();
      continue;
    }
    if (hipMemcpy((i == 0 ? ref : out).data(), args->y, ybytes, hipMemcpyDeviceToHost) !=
        hipSuccess) {
      st = FCONV_ERR_DEVICE;
      break;
    }
    if (i > 0 && fconv::output_difference(p, ref, out) > tol) continue;
    bool ok = hipEventRecord(e0, s) == hipSuccess;
    for (int r = 0; ok && r < repeats; ++r) ok = fconv::launch_conv(&q, a, s) == hipSuccess;
    ok = ok && hipEventRecord(e1, s) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
    float ms = 0.0f;
    if (!ok || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
      st = FCONV_ERR_DEVICE;
      break;
    }
    if (best < 0.0f || ms < best) {
      best = ms;
      best_i = i;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st != FCONV_OK) return st;
  fconv::apply_config(p, cand[best_i]);
  fconv::cache_store(p->d, cand[best_i]);
  if (best_us) *best_us = best * 1000.0f / static_cast<float>(repeats);
  // Leave y holding the chosen configuration's result.
  if (fconv::launch_conv(p, a, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
    return FCONV_ERR_DEVICE;
  return FCONV_OK;
}

}  // extern "C"
