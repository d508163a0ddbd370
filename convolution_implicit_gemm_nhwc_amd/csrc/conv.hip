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
  int32_t use_side, use_bias, use_bn, relu;
};

// ------------------------------------------------------------ filter repack

// HWIO [R][S][C][K] (= [Kg][K]) -> packed [Kp][KgP], rows in the permuted
// channel order above, reduction contiguous, zero-filled past K and Kg.
// One thread per 16-byte chunk of the packed filter.
template <int DT>
__global__ __launch_bounds__(256) void pack_filter_kernel(const void* __restrict__ w_,
                                                          void* __restrict__ wp_,
                                                          int32_t K, int32_t Kg,
                                                          int32_t KgP, int32_t Kp) {
  using T = typename Dt<DT>::T;
  constexpr int E = Dt<DT>::kChunk;
  const T* w = static_cast<const T*>(w_);
  T* wp = static_cast<T*>(wp_);
  const int chunks_per_row = KgP / E;
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
  *reinterpret_cast<i32x4*>(wp + static_cast<int64_t>(p) * KgP + q * E) = u.v;
}

// ---------------------------------------------------------------- epilogues

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// int8: TensorFlow conv_ops_fused_int8.cc, BiasActivationOutputKernel (cuDNN 8
// order).  v[e] is the int32 accumulator of channel ch0 + e.
__device__ inline void epilogue_store_i8(const int32_t (&v)[16], const ConvArgs& a,
                                         int m, int ch0, bool kvec) {
  int8_t* y = static_cast<int8_t*>(a.y) + static_cast<int64_t>(m) * a.K + ch0;
  const int8_t* side = a.use_side ? a.side + static_cast<int64_t>(m) * a.K + ch0 : nullptr;
  union {
    int8_t b[16];
    i32x4 v;
  } s, o;
  if (side) {
    if (kvec) {
      s.v = *reinterpret_cast<const i32x4*>(side);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) s.b[e] = (ch0 + e < a.K) ? side[e] : int8_t(0);
    }
  }
  const float lo = a.relu ? 0.0f : -128.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int ch = ch0 + e;
    const float b = (kvec || ch < a.K) ? a.bias[ch] : 0.0f;
    float t = static_cast<float>(v[e]);        // int32 -> fp32, nearest even
    t = t * a.cis;                             // (1) scale
    if (side) t = __builtin_fmaf(static_cast<float>(s.b[e]), a.sis, t);  // (2)
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
  const T* __restrict__ wrow = static_cast<const T*>(a.wp) +
                               static_cast<int64_t>(blockIdx.y * kTileN + col) * a.KgP +
                               g * E;
  const int64_t tile_stride = static_cast<int64_t>(16) * a.KgP;

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
    epilogue_store_i8(v, a, m, ch0, KVEC);
  } else {
    float v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * j + i] = acc[j][i];
    epilogue_store_float<DT>(v, a, m, ch0, KVEC);
  }
}

// ------------------------------------------------------------- dispatch

template <int DT>
hipError_t launch_pack(const fconv_plan_s* p, const void* w, void* wp, hipStream_t s) {
  const int64_t chunks = static_cast<int64_t>(p->Kp) * (p->KgP / p->chunk_elems);
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

hipError_t launch_pack_any(const fconv_plan_s* p, const void* w, void* wp, hipStream_t s) {
  switch (p->d.dtype) {
    case FCONV_INT8: return launch_pack<FCONV_INT8>(p, w, wp, s);
    case FCONV_BF16: return launch_pack<FCONV_BF16>(p, w, wp, s);
    default: return launch_pack<FCONV_FP32>(p, w, wp, s);
  }
}

hipError_t launch_conv(const fconv_plan_s* p, const ConvArgs& a, hipStream_t s) {
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
  // TensorFlow's output kernel skips the side input when its scale is zero.
  a.use_side = p->op_side && args->side_input_scale != 0.0f;
  a.use_bias = p->op_bias;
  a.use_bn = p->op_bn;
  a.relu = p->op_relu;
  if (fconv::launch_conv(p, a, s) != hipSuccess) return FCONV_ERR_DEVICE;
  return FCONV_OK;
}

}  // extern "C"
