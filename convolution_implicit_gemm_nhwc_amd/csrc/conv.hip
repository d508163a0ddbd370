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

#include "plan.h"

namespace fconv {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
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

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Side-input chunk of output pixel m, channels ch0 .. ch0+15 (zero past K).
__device__ inline i32x4 load_side_chunk(const ConvArgs& a, int m, int ch0, bool kvec) {
  const int8_t* side = a.side + static_cast<int64_t>(m) * a.K + ch0;
  if (kvec) return *reinterpret_cast<const i32x4*>(side);
  union {
    int8_t b[16];
    i32x4 v;
  } s;
#pragma unroll
  for (int e = 0; e < 16; ++e) s.b[e] = (ch0 + e < a.K) ? side[e] : int8_t(0);
  return s.v;
}

// int8: TensorFlow conv_ops_fused_int8.cc, BiasActivationOutputKernel (cuDNN 8
// order).  v[e] is the int32 accumulator of channel ch0 + e; side_chunk holds
// the int8 side input of the same 16 channels (ignored unless a.use_side).
__device__ inline void epilogue_store_i8(const int32_t (&v)[16], const ConvArgs& a,
                                         int m, int ch0, bool kvec, i32x4 side_chunk) {
  int8_t* y = static_cast<int8_t*>(a.y) + static_cast<int64_t>(m) * a.K + ch0;
  union {
    int8_t b[16];
    i32x4 v;
  } s, o;
  s.v = side_chunk;
  const float lo = a.relu ? 0.0f : -128.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int ch = ch0 + e;
    const float b = (kvec || ch < a.K) ? a.bias[ch] : 0.0f;
    float t = static_cast<float>(v[e]);        // int32 -> fp32, nearest even
    t = t * a.cis;                             // (1) scale
    if (a.use_side) t = __builtin_fmaf(static_cast<float>(s.b[e]), a.sis, t);  // (2)
    t = t + b;                                 // (3) bias
    t = __builtin_rintf(t);                    // round half to even
    t = __builtin_fminf(__builtin_fmaxf(t, lo), 127.0f);
    o.b[e] = static_cast<int8_t>(static_cast<int32_t>(t));
  }
  if (kvec) {
    *reinterpret_cast<i32x4*>(y) = o.v;
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (ch0 + e < a.K) y[e] = o.b[e];
  }
}

// bf16 / fp32: bias -> batch-norm inference -> ReLU (MIOpen's CBNA order).
template <int DT>
__device__ inline void epilogue_store_float(const float (&v)[16], const ConvArgs& a,
                                            int m, int ch0, bool kvec) {
  float t[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int ch = ch0 + e;
    const bool live = kvec || ch < a.K;
    float x = v[e];
    if (a.use_bias && live) x = x + a.bias[ch];
    if (a.use_bn && live) {
      const float sc = a.bn_gamma[ch] / __builtin_sqrtf(a.bn_var[ch] + a.bn_eps);
      x = (x - a.bn_mean[ch]) * sc + a.bn_beta[ch];
    }
    if (a.relu) x = __builtin_fmaxf(x, 0.0f);
    t[e] = x;
  }
  const int64_t off = static_cast<int64_t>(m) * a.K + ch0;
  if constexpr (DT == FCONV_FP32) {
    float* y = static_cast<float*>(a.y) + off;
    if (kvec) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(y + 4 * q) = f32x4{t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]};
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (ch0 + e < a.K) y[e] = t[e];
    }
  } else {
    uint16_t* y = static_cast<uint16_t*>(a.y) + off;
    union {
      uint16_t h[16];
      i32x4 v[2];
    } o;
#pragma unroll
    for (int e = 0; e < 16; ++e) o.h[e] = f32_to_bf16_rne(t[e]);
    if (kvec) {
      reinterpret_cast<i32x4*>(y)[0] = o.v[0];
      reinterpret_cast<i32x4*>(y)[1] = o.v[1];
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (ch0 + e < a.K) y[e] = o.h[e];
    }
  }
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
    for (int kk = 0; kk < a.KgP; kk += KSTEP) {
      const i32x4 b = gather_patch_chunk<DT, MODE>(xn, a, mvalid, hbase, wbase, kk + g * E);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const i32x4 w4 = *reinterpret_cast<const i32x4*>(wrow + j * tile_stride + kk);
        acc[j] = mma_chunk(w4, b, acc[j], static_cast<Dt<DT>*>(nullptr));
      }
    }
  }

  const int ch0 = blockIdx.y * kTileN + 16 * g;
  if (!mvalid || ch0 >= a.K) return;
  if constexpr (DT == FCONV_INT8) {
    int32_t v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * j + i] = acc[j][i];
    const i32x4 sc = a.use_side ? load_side_chunk(a, m, ch0, KVEC) : i32x4{0, 0, 0, 0};
    epilogue_store_i8(v, a, m, ch0, KVEC, sc);
  } else {
    float v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * j + i] = acc[j][i];
    epilogue_store_float<DT>(v, a, m, ch0, KVEC);
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
// tile: 128 pixels x 128 output channels, 4 waves in a 2 x 2 grid of 64 x 64.
// The reduction advances in stages of 128 bytes (one filter tap, 128 bytes of
// its channels; two MFMA k-steps).  Per stage every thread fetches 4 pixel-row
// and 4 filter-row pieces of 16 bytes with buffer loads -- taps in the
// padding and rows past M or Kp read zeros -- two stages ahead into a
// register ring, and writes a fetched stage into one half of a double-buffered
// LDS area.  LDS rows are 144 bytes (128 + 16 pad, an odd multiple of 16):
// the 16 rows one ds_read_b128 touches fall in distinct bank groups.  Each
// wave does a 4 x 4 grid of 16x16 MFMAs per k-step: 8 fragment reads feed 16
// MFMAs.
constexpr int kTileBM = 128, kTileBN = 128, kTileStage = 128, kTileRow = kTileStage + 16;

template <int DT, bool KVEC>
__global__ __launch_bounds__(kThreads) void conv_tile_kernel(ConvArgs a) {
  using Acc = typename Dt<DT>::Acc;
  constexpr int E = Dt<DT>::kChunk;
  constexpr int ES = 16 / E;
  constexpr int SE = kTileStage / ES;  // reduction elements per stage
  __shared__ __attribute__((aligned(16))) char lds[2][(kTileBM + kTileBN) * kTileRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int g = lane >> 4, col = lane & 15;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.wp, a.wp_bytes);

  // Loader role: rows r0 + 32h (h = 0..3) of both tiles, 16-byte piece q.
  const int q = tid & 7;
  const int r0 = tid >> 3;
  int hb[4], wb[4], pbase[4];
  uint32_t wbase[4];
  const int RS = a.wrow_bytes;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int m = blockIdx.x * kTileBM + r0 + 32 * h;
    const int mm = m < a.M ? m : 0;
    const uint32_t qq = fast_div(static_cast<uint32_t>(mm), a.wo_mul, a.wo_add, a.wo_shift);
    const int wo = mm - static_cast<int>(qq) * a.Wo;
    const uint32_t n = fast_div(qq, a.ho_mul, a.ho_add, a.ho_shift);
    const int ho = static_cast<int>(qq) - static_cast<int>(n) * a.Ho;
    hb[h] = m < a.M ? ho * a.sh - a.pt : -(1 << 20);
    wb[h] = wo * a.sw - a.pl;
    pbase[h] = static_cast<int>(n) * a.H * a.W * a.C * ES + q * 16;
    wbase[h] = static_cast<uint32_t>((blockIdx.y * kTileBN + r0 + 32 * h) * RS + q * 16);
  }

  const int cs = a.C / SE;  // stages per filter tap
  const int nst = a.R * a.S * cs;
  auto fetch = [&](int st, i32x4(&px)[4], i32x4(&fl)[4]) {
    const int tap = st / cs;
    const int c0b = (st - tap * cs) * kTileStage;
    const int r = tap / a.S;
    const int s = tap - r * a.S;
    const bool live = st < nst;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int hi = hb[h] + r, wi = wb[h] + s;
      const bool ok = live && static_cast<unsigned>(hi) < static_cast<unsigned>(a.H) &&
                      static_cast<unsigned>(wi) < static_cast<unsigned>(a.W);
      const uint32_t off =
          ok ? static_cast<uint32_t>(pbase[h] + (hi * a.W + wi) * a.C * ES + c0b) : kOutOfRange;
      px[h] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
      fl[h] = __builtin_amdgcn_raw_buffer_load_b128(
          wr, live ? wbase[h] + st * kTileStage : kOutOfRange, 0, 0);
    }
  };
  auto stash = [&](int buf, const i32x4(&px)[4], const i32x4(&fl)[4]) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      *reinterpret_cast<i32x4*>(&lds[buf][(r0 + 32 * h) * kTileRow + q * 16]) = px[h];
      *reinterpret_cast<i32x4*>(&lds[buf][(kTileBM + r0 + 32 * h) * kTileRow + q * 16]) = fl[h];
    }
  };

  Acc acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = Acc{0, 0, 0, 0};

  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const char* pl = &lds[buf][(wm * 64 + col) * kTileRow + kk * 64 + g * 16];
      const char* fb = &lds[buf][(kTileBM + wn * 64 + col) * kTileRow + kk * 64 + g * 16];
      i32x4 pf[4], ff[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pf[i] = *reinterpret_cast<const i32x4*>(pl + i * 16 * kTileRow);
#pragma unroll
      for (int j = 0; j < 4; ++j) ff[j] = *reinterpret_cast<const i32x4*>(fb + j * 16 * kTileRow);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = mma_chunk(ff[j], pf[i], acc[i][j], static_cast<Dt<DT>*>(nullptr));
    }
  };

  // Two stages of loads in flight (registers A and B alternate), one stage
  // being computed from LDS.
  // Stages go in pairs with no exit in between (one back-edge keeps the
  // accumulators in place); fetches past the last stage read zeros.
  i32x4 pxA[4], flA[4], pxB[4], flB[4];
  fetch(0, pxA, flA);
  fetch(1, pxB, flB);
  stash(0, pxA, flA);
  __syncthreads();
  for (int st = 0; st + 2 <= nst; st += 2) {
    fetch(st + 2, pxA, flA);
    compute(0);          // stage st
    stash(1, pxB, flB);  // stage st+1
    __syncthreads();
    fetch(st + 3, pxB, flB);
    compute(1);          // stage st+1
    stash(0, pxA, flA);  // stage st+2
    __syncthreads();
  }
  if (nst & 1) compute(0);  // the last stage, already in buffer 0

  const int ch0 = blockIdx.y * kTileBN + wn * 64 + 16 * g;
  if (ch0 >= a.K) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = blockIdx.x * kTileBM + wm * 64 + i * 16 + col;
    if (m >= a.M) continue;
    if constexpr (DT == FCONV_INT8) {
      int32_t v[16];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * j + e] = acc[i][j][e];
      const i32x4 sc = a.use_side ? load_side_chunk(a, m, ch0, KVEC) : i32x4{0, 0, 0, 0};
      epilogue_store_i8(v, a, m, ch0, KVEC, sc);
    } else {
      float v[16];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * j + e] = acc[i][j][e];
      epilogue_store_float<DT>(v, a, m, ch0, KVEC);
    }
  }
}

// ------------------------------------------------------- streaming conv

// Requantisation of one output, cuDNN 8 order (TensorFlow conv_ops_fused_int8.cc,
// BiasActivationOutputKernel): (float)acc * cis, + side * sis as one fused
// multiply-add, + bias, each an fp32 operation.  Round half to even and clip
// are done together: adding 1.5 * 2^23 rounds t to the nearest integer (ties
// to even) into the low mantissa bits, exactly for |t| < 2^22, and monotonically
// beyond, where the clip saturates anyway; a med3 against the two biased
// bounds clips, and the low byte of the result's bit pattern is then the int8
// value (two's complement).  Checked exhaustively over every finite fp32 t.
// `lo_b` / `hi_b` are 1.5*2^23 + (ReLU ? 0 : -128) and 1.5*2^23 + 127.
constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23
template <bool SIDE>
__device__ inline uint32_t requant_i8_bits(int32_t acc, int8_t side, float bias, float cis,
                                           float sis, float lo_b, float hi_b) {
  float v = static_cast<float>(acc);  // int32 -> fp32, nearest even
  v = v * cis;                        // (1) scale
  if constexpr (SIDE) v = __builtin_fmaf(static_cast<float>(side), sis, v);  // (2) side
  v = v + bias;                       // (3) bias
  v = v + kRoundMagic;                // round half to even
  v = __builtin_amdgcn_fmed3f(v, lo_b, hi_b);  // clip
  return __builtin_bit_cast(uint32_t, v);
}
// Low bytes of two / of two pairs packed with v_perm_b32.
__device__ inline uint32_t pack_pair(uint32_t lo_val, uint32_t hi_val) {
  return __builtin_amdgcn_perm(hi_val, lo_val, 0x0c0c0400u);  // [lo.b0, hi.b0, 0, 0]
}
__device__ inline uint32_t pack_word(uint32_t lo_pair, uint32_t hi_pair) {
  return __builtin_amdgcn_perm(hi_pair, lo_pair, 0x05040100u);  // [lo.b0, lo.b1, hi.b0, hi.b1]
}

// int8 epilogue of one 16-pixel tile for this lane's pixel and 16 channels,
// written with one buffer store; an out-of-range offset drops it.
template <bool SIDE>
__device__ inline void stream_epilogue_i8(const i32x4 (&acc)[4], i32x4 side_chunk,
                                          const float (&bias)[16], float cis, float sis,
                                          float lo_b, float hi_b, __amdgpu_buffer_rsrc_t yr,
                                          uint32_t off) {
  union {
    int8_t b[16];
    i32x4 v;
  } sd;
  sd.v = side_chunk;
  uint32_t packed[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t vb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vb[i] = requant_i8_bits<SIDE>(acc[j][i], sd.b[4 * j + i], bias[4 * j + i], cis, sis,
                                    lo_b, hi_b);
    packed[j] = pack_word(pack_pair(vb[0], vb[1]), pack_pair(vb[2], vb[3]));
  }
  __builtin_amdgcn_raw_buffer_store_b128(
      i32x4{static_cast<int32_t>(packed[0]), static_cast<int32_t>(packed[1]),
            static_cast<int32_t>(packed[2]), static_cast<int32_t>(packed[3])},
      yr, off, 0, 0);
}

// Streaming kernel for int8 layers with a short reduction: R x S taps of CS
// k-steps (64 channels each).  Persistent: one workgroup per CU.  Each wave
// keeps its 64-channel slice of the packed filter in registers for the whole
// kernel (no LDS traffic) and walks a contiguous range of 16-pixel tiles;
// workgroup ranges are grouped by XCD so neighbouring tiles, which share
// input rows, share an L2.  Per tile, the patch fragments of all k-steps are
// buffer loads issued two tiles ahead; a tap outside the image gets an
// offset past the extent and reads zeros.  Each iteration issues the current
// tile's MFMAs and, in the same basic block, the previous tile's epilogue,
// so the matrix cores and the VALU work overlap.  Offsets use 24-bit
// multiplies (every operand and product here is far below 2^24 / 2^31).
template <int R, int S, int CS, bool SIDE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void conv_stream_i8_kernel(ConvArgs a) {
  constexpr int NKS = R * S * CS;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int col = lane & 15;
  const int ch0 = blockIdx.y * 64 + 16 * g;

  const int G = gridDim.x;
  const int bx = blockIdx.x;
  const int b = (G % 8 == 0) ? (bx % 8) * (G / 8) + bx / 8 : bx;
  const int t_begin = b * a.tiles / G;  // b * tiles < 2^31 (checked at plan time)
  const int t_end = (b + 1) * a.tiles / G;
  const int n_tiles = t_end - t_begin - wave > 0 ? (t_end - t_begin - wave + 3) / 4 : 0;

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
  // falls outside the image or the tile outside this wave's range).
  auto offsets = [&](int k, uint32_t(&o)[NKS]) {
    const int t = t_begin + wave + 4 * k;
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
  // Output (and side-input) offset of tile k for this lane, or out of range;
  // the uniform range test is folded into one unsigned compare.
  auto out_off = [&](int k) -> uint32_t {
    const int m = (t_begin + wave + 4 * k) * 16 + col;
    const bool ok = static_cast<unsigned>(k) < static_cast<unsigned>(n_tiles) &&
                    m < a.M && ch0 < a.K;
    return ok ? static_cast<uint32_t>(__mul24(m, a.K) + ch0) : kOutOfRange;
  };
  auto issue_side = [&](int k) -> i32x4 {
    if constexpr (SIDE) return __builtin_amdgcn_raw_buffer_load_b128(sr, out_off(k), 0, 0);
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
  // global->LDS copy of its 64 padded rows, then every wave reads its
  // fragments for all k-steps and the 4 MFMA tiles into registers.  The 16
  // bias values of this lane's channels come in with four buffer loads
  // (channels past K read 0).
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int RS = a.wrow_bytes;
  {
    const char* src = static_cast<const char*>(a.wp) + static_cast<int64_t>(blockIdx.y) * 64 * RS;
    for (int i = wave; i < RS / 16; i += 4)
      __builtin_amdgcn_global_load_lds(src + i * 1024 + lane * 16,
                                       (lds_ptr_t)(smem + i * 1024), 16, 0, 0);
  }
  const __amdgpu_buffer_rsrc_t br = make_rsrc(a.bias, static_cast<uint32_t>(a.K) * 4u);
  float bias[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 v = __builtin_bit_cast(
        f32x4, __builtin_amdgcn_raw_buffer_load_b128(br, static_cast<uint32_t>((ch0 + 4 * q) * 4), 0, 0));
    bias[4 * q] = v.x;
    bias[4 * q + 1] = v.y;
    bias[4 * q + 2] = v.z;
    bias[4 * q + 3] = v.w;
  }
  const float cis = a.cis, sis = a.sis;
  const float lo_b = kRoundMagic + (a.relu ? 0.0f : -128.0f), hi_b = kRoundMagic + 127.0f;
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt = expcnt = lgkmcnt = 0
  __syncthreads();
  i32x4 Wf[NKS][4];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      Wf[ks][j] = *reinterpret_cast<const i32x4*>(smem + (j * 16 + col) * RS + ks * 64 + g * 16);

  i32x4 accA[4], accB[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) accB[j] = zero4;

  // One half of a loop trip, software-pipelined by hand: the MFMAs of the
  // tile in bX (into accX) are split by k-step into NKS chunks; each chunk
  // also issues that k-step's refill load for tile k_load and finishes EPC of
  // the 16 epilogue outputs of the previous tile (accY, side sY).  A
  // scheduling barrier closes each chunk, so the VALU epilogue runs under the
  // matrix-core work instead of before or after it.
  constexpr int EPC = (16 + NKS - 1) / NKS;
  auto half = [&](i32x4(&bX)[NKS], i32x4(&accX)[4], const i32x4(&accY)[4], i32x4 sY,
                  int k_load, uint32_t off_prev) {
    uint32_t o[NKS];
    offsets(k_load, o);
    union {
      int8_t b[16];
      i32x4 v;
    } sd;
    sd.v = sY;
    uint32_t pairs[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    uint32_t words[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        accX[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(Wf[ks][j], bX[ks],
                                                        ks == 0 ? zero4 : accX[j], 0, 0, 0);
      bX[ks] = __builtin_amdgcn_raw_buffer_load_b128(xr, o[ks], 0, 0);
      // EPC is even, so a chunk finishes whole pairs of outputs.
#pragma unroll
      for (int e = ks * EPC; e < (ks + 1) * EPC && e < 16; e += 2) {
        const uint32_t v0 = requant_i8_bits<SIDE>(accY[e / 4][e % 4], sd.b[e], bias[e], cis,
                                                  sis, lo_b, hi_b);
        const uint32_t v1 = requant_i8_bits<SIDE>(accY[e / 4][e % 4 + 1], sd.b[e + 1],
                                                  bias[e + 1], cis, sis, lo_b, hi_b);
        pairs[e / 2] = pack_pair(v0, v1);
        if (e % 4 == 2) words[e / 4] = pack_word(pairs[e / 2 - 1], pairs[e / 2]);
      }
      // Pin this chunk's outputs here: without it the arithmetic, which has
      // no memory effects, is sunk to the store at the end of the half.
      asm volatile("" : "+v"(words[0]), "+v"(words[1]), "+v"(words[2]), "+v"(words[3]),
                   "+v"(pairs[0]), "+v"(pairs[2]), "+v"(pairs[4]), "+v"(pairs[6]));
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_raw_buffer_store_b128(
        i32x4{static_cast<int32_t>(words[0]), static_cast<int32_t>(words[1]),
              static_cast<int32_t>(words[2]), static_cast<int32_t>(words[3])},
        yr, off_prev, 0, 0);
  };

  // Two tiles per trip and no exit in between, so both halves see the same
  // memory-operation history: half A computes tile k and finishes tile k-1,
  // half B computes tile k+1 and finishes tile k.  A tile past the wave's
  // range loads zeros and its store is dropped.
  int k = 0;
  for (; k < n_tiles; k += 2) {
    half(bA, accA, accB, sB, k + 2, out_off(k - 1));
    sB = issue_side(k + 1);
    half(bB, accB, accA, sA, k + 3, out_off(k));
    sA = issue_side(k + 2);
  }
  stream_epilogue_i8<SIDE>(accB, sB, bias, cis, sis, lo_b, hi_b, yr, out_off(k - 1));
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

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int R, int S, int CS>
hipError_t launch_stream_shape(const fconv_plan_s* p, const ConvArgs& a, hipStream_t s) {
  const int cus = device_cu_count();
  int grid = (a.tiles + 3) / 4;  // at least one tile per wave
  if (grid > cus) grid = cus;
  const dim3 g(static_cast<unsigned>(grid), static_cast<unsigned>(p->Kp / 64));
  const size_t lds = static_cast<size_t>(64) * a.wrow_bytes;
  if (a.use_side)
    hipLaunchKernelGGL((conv_stream_i8_kernel<R, S, CS, true>), g, dim3(kThreads), lds, s, a);
  else
    hipLaunchKernelGGL((conv_stream_i8_kernel<R, S, CS, false>), g, dim3(kThreads), lds, s, a);
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
  hipLaunchKernelGGL((conv_tile_kernel<DT, true>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_conv(const fconv_plan_s* p, const ConvArgs& a, hipStream_t s) {
  if (p->variant == kStream) return launch_stream(p, a, s);
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
  fconv::ConvArgs a;
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
  a.wp_bytes = static_cast<uint32_t>(p->ws_bytes);
  a.tiles = static_cast<int32_t>((p->M + 15) / 16);
  a.wo_mul = p->wo_div.mul; a.wo_add = p->wo_div.add; a.wo_shift = p->wo_div.shift;
  a.ho_mul = p->ho_div.mul; a.ho_add = p->ho_div.add; a.ho_shift = p->ho_div.shift;
  // TensorFlow's output kernel skips the side input when its scale is zero.
  a.use_side = p->op_side && args->side_input_scale != 0.0f;
  a.use_bias = p->op_bias;
  a.use_bn = p->op_bn;
  a.relu = p->op_relu;
  if (fconv::launch_conv(p, a, s) != hipSuccess) return FCONV_ERR_DEVICE;
  return FCONV_OK;
}

}  // extern "C"
