// Weight gradient of the NHWC convolution on gfx950 (CDNA4), and its C ABI.
//
//   dw[r,s,c,k] = sum over pixels m = (n, ho, wo) of P[m, (r,s,c)] * dy[m, k]
//   P[m, (r,s,c)] = X(n, ho*sh - pt + r, wo*sw - pl + s, c)   (zero outside)
//
// TensorFlow conv_grad_filter_ops.cc (Conv2DCustomBackpropFilterOp) forms,
// per image, the Im2col patch matrix [Ho*Wo, R*S*C] and multiplies its
// transpose by the output gradient [Ho*Wo, K].  Here the sum over images is
// folded into one implicit GEMM whose reduction runs over all M = N*Ho*Wo
// pixels:
//   rows   k  = output channel          K
//   cols   kk = (r, s, c)               Kg = R*S*C   (HWIO row order)
//   reduction m = (n, ho, wo)           M
// The patch matrix is never built: each lane gathers 16-byte slices of
// patch rows straight from the NHWC input (taps in the padding read zero).
//
// Matrix-core mapping.  The 16x16 MFMA wants, per lane, a 16-byte run of the
// reduction index for one row (A) and one column (B).  Both operands arrive
// pixel-major (NHWC: the channels of one pixel are contiguous), so every
// fragment needs a transpose.  A = dy (rows k), B = patch (cols kk), so a
// lane ends with 4 consecutive output channels of one (r, s, c): one
// 16-byte store.  Two kernels:
//  - wgrad_dma_kernel (C and K multiples of the 16-byte chunk): both
//    operands are copied buffer->LDS in their natural layout, and bf16
//    fragments come from gfx950's transposed LDS read; fp32 fragments hold
//    one element per lane and need no transpose.
//  - wgrad_kernel (any shape; also under FCONV_WGRAD_KERNEL=staged): a lane
//    fetches the same 16-byte channel chunk of E consecutive pixels (E = 8
//    bf16 / 4 fp32) into registers, transposes the E x E block and writes E
//    pixel runs, one per channel, to LDS rows of 128 bytes; fragment reads
//    are then single ds_read_b128s.
//
// Work split.  A workgroup owns a TK x 128 tile of dw over one range of
// pixels.  When tiles alone do not fill the chip, the pixels are split into
// ranges; each range writes its fp32 partial tile to the workspace and a
// second kernel adds the ranges in a fixed order, so the result does not
// depend on scheduling.  Workgroups of one range are placed on one XCD
// (blockIdx round-robins over the 8 XCDs), so the range's input and gradient
// rows are fetched into one L2 and shared by all its tiles.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdint.h>

#include <limits.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "plan.h"

struct fconv_wgrad_plan_s {
  fconv_desc d;
  int32_t Ho, Wo, pt, pb, pl, pr;
  int32_t esize;     // bytes per x / dy element
  int32_t E;         // elements per 16-byte chunk
  int64_t M;         // N*Ho*Wo, reduction length
  int32_t Kg;        // R*S*C
  bool out_fp32;     // dw written as fp32
  bool vec;          // C % E == 0 and K % E == 0: 16-byte gathers
  bool dma;          // vec shapes: the direct-to-LDS kernel (else register-staged)
  int32_t ring;      // direct-to-LDS kernel: stages in its LDS ring (4 or 8)
  int32_t tk;        // output channels per tile (64, 128, or 256 with 8 waves)
  bool ksplit;       // bf16 4-stage ring, 64/128-channel tile: two wave groups split each range
  bool halo;         // bf16 3x3 stride 1: the row-halo kernel (ranges of output rows)
  int32_t rps;       // row-halo kernel: output rows per step (2 when Wo <= 32, else 1)
  int32_t tiles_k, tiles_kk;
  int32_t splits;    // pixel ranges
  int32_t m_per_split;
  int64_t lp;        // partial tile stride in floats (Kg*K rounded up to 4)
  size_t ws_bytes;
  int64_t x_elems, dy_elems, dw_elems;
  fconv::FastDiv hw_div, wo_div, ho_div;
  const char* kernel_name;
};

namespace fconv {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWgThreads = 256;   // register-staged kernel: 4 waves
constexpr int kWgTKK = 128;       // (r,s,c) columns per tile
constexpr int kWgRowBytes = 128;  // one LDS row: 8 slots of 16 bytes
constexpr int kWgTargetBlocks = 512;  // two workgroups per CU (256 CUs)
constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past every extent: reads 0
constexpr int kBufferDword3 = 0x00020000;      // raw buffer descriptor, gfx9 family

struct WgArgs {
  const void* x;
  const void* dy;
  void* out;  // partial sums [split][lp] fp32, or dw
  int32_t N, H, W, C, K, R, S, sh, sw, pt, pl, Ho, Wo;
  int32_t M, Kg;
  int32_t tiles_k, tiles_kk, splits, m_per_split;
  int32_t blocks;  // splits * tiles_k * tiles_kk
  int32_t out_mode;  // 0 partial fp32, 1 dw fp32, 2 dw bf16
  int64_t lp;
  uint32_t x_bytes, dy_bytes;
  uint32_t hw_mul, hw_add, hw_shift, wo_mul, wo_add, wo_shift;
  int32_t wo_ge_e;  // Wo >= pixels per gather group: one wrap at most
  uint32_t ho_mul, ho_add, ho_shift;  // row-halo kernel: output row / Ho
};

__device__ inline uint32_t fast_div(uint32_t n, uint32_t mul, uint32_t add, uint32_t shift) {
  return (__umulhi(n, mul) + (add ? n : 0u)) >> shift;
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kBufferDword3);
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  // Hardware round to nearest even (v_cvt_pk_bf16_f32), NaN kept quiet:
  // identical on all 2^32 inputs to the integer form of the same rounding.
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// One 16-byte fragment pair through the matrix core: 8 bf16 per lane (one
// instruction) or 4 fp32 per lane (four instructions, one element each).
template <int DT>
__device__ inline f32x4 wg_mma(i32x4 a, i32x4 b, f32x4 c) {
  if constexpr (DT == FCONV_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    // Bit-cast whole vectors, then index (a bit-cast of one ext-vector
    // element reads element 0 in this compiler).
    const f32x4 af = __builtin_bit_cast(f32x4, a);
    const f32x4 bf = __builtin_bit_cast(f32x4, b);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af.x, bf.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af.y, bf.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af.z, bf.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af.w, bf.w, c, 0, 0, 0);
    return c;
  }
}

// Slot of pixel run `chunk` in LDS row `row`.  Rows are 128 bytes; the
// xor with the row's low bits spreads the 16 rows one fragment read touches
// over all eight slots, and the xor with bits 3..5 does the same for the
// rows one transposed write touches (E apart).
__device__ inline int wg_slot(int row, int chunk) {
  return chunk ^ ((row ^ (row >> 3)) & 7);
}

// Store a wave's accumulators: lane holds D[k][kk] for k = k0 + 64 wk +
// 16 i + 4 g + t (t = 0..3) and kk = kk0 + wkk * 16 NJ + 16 j + lane % 16; to
// the pixel range's partial tile (fp32) or straight to dw (fp32 or bf16).
template <int NI, int NJ>
__device__ inline void wg_store(const WgArgs& a, const f32x4 (&acc)[NI][NJ], int split, int k0,
                                int kk0, int wk, int wkk, int lane) {
  const int g = lane >> 4;
  const bool kvec4 = (a.K & 3) == 0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int k = k0 + wk * 64 + 16 * i + 4 * g;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int kk = kk0 + wkk * (NJ * 16) + 16 * j + (lane & 15);
      if (kk >= a.Kg || k >= a.K) continue;
      const f32x4 v = acc[i][j];
      const int64_t base = static_cast<int64_t>(kk) * a.K + k;
      if (a.out_mode == 0) {
        float* o = static_cast<float*>(a.out) + split * a.lp + base;
        if (kvec4) {
          *reinterpret_cast<f32x4*>(o) = v;
        } else {
          for (int t = 0; t < 4 && k + t < a.K; ++t) o[t] = v[t];
        }
      } else if (a.out_mode == 1) {
        float* o = static_cast<float*>(a.out) + base;
        if (kvec4) {
          *reinterpret_cast<f32x4*>(o) = v;
        } else {
          for (int t = 0; t < 4 && k + t < a.K; ++t) o[t] = v[t];
        }
      } else {
        uint16_t* o = static_cast<uint16_t*>(a.out) + base;
        if (kvec4) {
          const uint32_t lo = f32_to_bf16_rne(v[0]) | (uint32_t(f32_to_bf16_rne(v[1])) << 16);
          const uint32_t hi = f32_to_bf16_rne(v[2]) | (uint32_t(f32_to_bf16_rne(v[3])) << 16);
          *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
        } else {
          for (int t = 0; t < 4 && k + t < a.K; ++t) o[t] = f32_to_bf16_rne(v[t]);
        }
      }
    }
  }
}

// Main kernel.  DT: bf16 or fp32.  TK: output channels per tile (64 / 128).
// VEC: C and K are multiples of E, so every gathered chunk is one 16-byte
// load; otherwise elements are gathered one by one (any shape).
//
// Per stage (BM = 8*E pixels) every thread fetches its tasks' chunks (one
// task = one 16-byte column chunk x E consecutive pixels, of dy or of the
// patch matrix), transposes them in registers and writes them to the stage's
// LDS buffer; after one barrier the four waves (a 2x2 or 1x4 grid over the
// tile) run the stage's MFMAs.  Loads run two stages ahead (two register
// sets), LDS holds two stages.  The patch gather costs more VALU work than
// the dy gather, so the two halves of the workgroup swap roles on odd
// stages: every SIMD then carries the same load.
template <int DT, int TK, bool VEC>
__global__ __launch_bounds__(kWgThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void wgrad_kernel(WgArgs a) {
  constexpr int ES = DT == FCONV_BF16 ? 2 : 4;
  constexpr int E = 16 / ES;
  constexpr int BM = 8 * E;                  // pixels per stage
  constexpr int ROWS = TK + kWgTKK;          // LDS rows per stage
  constexpr int STAGE_BYTES = ROWS * kWgRowBytes;
  constexpr int NT_DY = (TK / E) * 8;        // dy tasks per stage
  constexpr int NT = NT_DY + (kWgTKK / E) * 8;
  constexpr int TPT = (NT + kWgThreads - 1) / kWgThreads;  // tasks per thread
  constexpr int WK = TK / 64;                // waves along k (1 or 2)
  constexpr int WKK = 4 / WK;                // waves along kk (4 or 2)
  constexpr int NI = 4;                      // 16-row MFMA tiles per wave along k
  constexpr int NJ = kWgTKK / WKK / 16;      // along kk (2 or 4)

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE_BYTES];

  // Block -> (pixel range, tile).  Consecutive logical ids share a pixel
  // range; the remap puts consecutive ids on one XCD when the grid is a
  // multiple of 8 (the launcher pads it so).
  const int nb = gridDim.x;
  const int b = blockIdx.x;
  const int logical = (nb % 8 == 0) ? (b % 8) * (nb / 8) + b / 8 : b;
  if (logical >= a.blocks) return;
  const int tiles = a.tiles_k * a.tiles_kk;
  const int split = logical / tiles;
  const int tile = logical % tiles;
  const int k0 = (tile % a.tiles_k) * TK;
  const int kk0 = (tile / a.tiles_k) * kWgTKK;
  const int m_begin = split * a.m_per_split;
  const int m_end = min(a.M, m_begin + a.m_per_split);
  const int nst = (m_end - m_begin + BM - 1) / BM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wk = wave % WK, wkk = wave / WK;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t dr = make_rsrc(a.dy, a.dy_bytes);

  // Task constants of both roles (role p: task id (tid ^ 128p) + 256 i; the
  // xor swaps waves 0,1 with 2,3 and keeps every wave's tasks of one kind,
  // since the task counts are multiples of 64).
  struct Task {
    int on, isdy;   // wave-uniform
    int pm;         // first pixel of the task inside the stage (E * group)
    int col;        // first channel k (dy) or column kk (patch) of the chunk
    int dr, ds, c;  // patch: tap row/col offsets r - pt, s - pl and channel
    int laddr;      // LDS byte offset of the chunk's first row, | slot xor << 4
  };
  Task tk[2][TPT];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int t = (tid ^ (p ? 128 : 0)) + i * kWgThreads;
      Task& T = tk[p][i];
      T.on = t < NT;
      T.isdy = t < NT_DY;
      const int local = T.isdy ? t : t - NT_DY;
      const int ncc = (T.isdy ? TK : kWgTKK) / E;
      const int cc = local % ncc;
      const int pc = local / ncc;
      T.pm = pc * E;
      T.col = (T.isdy ? k0 : kk0) + cc * E;
      T.dr = T.ds = T.c = 0;
      if (!T.isdy && VEC) {
        const int rs = T.col / a.C;
        T.c = T.col - rs * a.C;
        const int r = rs / a.S;
        T.dr = r - a.pt;
        T.ds = rs - r * a.S - a.pl;
      }
      // Row of channel j of the chunk: row0 + j.  With row0 a multiple of E
      // (E = 4 or 8) the slot of pixel group pc in that row is
      // (pc ^ s0) ^ j, s0 the xor of row0 (see wg_slot); row0 * 128 has
      // bits 4..6 clear, so the slot bits can ride in those.
      const int row0 = (T.isdy ? 0 : TK) + cc * E;
      T.laddr = row0 * kWgRowBytes + ((pc ^ ((row0 ^ (row0 >> 3)) & 7)) << 4);
    }
  }

  // Element offset (in x) of the patch value of pixel m at tap (dr, ds),
  // channel c; -1 outside the image or past the pixel range.  Used by the
  // element-wise gather only.
  auto patch_elem = [&](int m, int dr, int ds, int c) -> int64_t {
    if (m >= m_end) return -1;
    const uint32_t n = fast_div(static_cast<uint32_t>(m), a.hw_mul, a.hw_add, a.hw_shift);
    const uint32_t rem = static_cast<uint32_t>(m) - n * static_cast<uint32_t>(a.Ho * a.Wo);
    const uint32_t ho = fast_div(rem, a.wo_mul, a.wo_add, a.wo_shift);
    const uint32_t wo = rem - ho * static_cast<uint32_t>(a.Wo);
    const int hi = static_cast<int>(ho) * a.sh + dr;
    const int wi = static_cast<int>(wo) * a.sw + ds;
    if (hi < 0 || hi >= a.H || wi < 0 || wi >= a.W) return -1;
    return ((static_cast<int64_t>(n) * a.H + hi) * a.W + wi) * a.C + c;
  };

  auto fetch = [&](int st, const Task (&tasks)[TPT], i32x4 (&R)[TPT][E]) {
    const int mb = m_begin + st * BM;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const Task& T = tasks[i];
      int m0 = mb + T.pm;
      // Opaque per stage: otherwise every pixel's offset becomes an
      // induction variable of the stage loop, and they do not fit in
      // registers.
      asm volatile("" : "+v"(m0));
      if constexpr (VEC) {
        uint32_t off[E];
        if (__builtin_amdgcn_readfirstlane(T.isdy)) {
          // dy rows are contiguous: pixel m0 + e at (m0 + e) * K + col.
          const bool ok = T.on && T.col < a.K;
          const uint32_t o0 = static_cast<uint32_t>((m0 * a.K + T.col) * ES);
          const uint32_t step = static_cast<uint32_t>(a.K * ES);
#pragma unroll
          for (int e = 0; e < E; ++e)
            off[e] = (ok && m0 + e < m_end) ? o0 + e * step : kOutOfRange;
        } else {
          const bool ok = T.on && T.col < a.Kg;
          // Decode the group's first pixel once; the others follow by
          // stepping wo (at most one wrap while Wo >= E).
          const uint32_t um0 = static_cast<uint32_t>(m0);
          const uint32_t n0 = fast_div(um0, a.hw_mul, a.hw_add, a.hw_shift);
          const uint32_t rem = um0 - n0 * static_cast<uint32_t>(a.Ho * a.Wo);
          const uint32_t ho0 = fast_div(rem, a.wo_mul, a.wo_add, a.wo_shift);
          const int wo0 = static_cast<int>(rem - ho0 * static_cast<uint32_t>(a.Wo));
#pragma unroll
          for (int e = 0; e < E; ++e) {
            int n = static_cast<int>(n0), ho = static_cast<int>(ho0), wo = wo0 + e;
            if (a.wo_ge_e) {
              const bool c1 = wo >= a.Wo;
              wo = c1 ? wo - a.Wo : wo;
              ho = ho + (c1 ? 1 : 0);
              const bool c2 = ho >= a.Ho;
              ho = c2 ? 0 : ho;
              n = n + (c2 ? 1 : 0);
            } else {
              const uint32_t um = um0 + e;
              const uint32_t nn = fast_div(um, a.hw_mul, a.hw_add, a.hw_shift);
              const uint32_t rr = um - nn * static_cast<uint32_t>(a.Ho * a.Wo);
              const uint32_t hh = fast_div(rr, a.wo_mul, a.wo_add, a.wo_shift);
              n = static_cast<int>(nn);
              ho = static_cast<int>(hh);
              wo = static_cast<int>(rr - hh * static_cast<uint32_t>(a.Wo));
            }
            const int hi = ho * a.sh + T.dr;
            const int wi = wo * a.sw + T.ds;
            const bool in = ok && m0 + e < m_end && static_cast<uint32_t>(hi) < static_cast<uint32_t>(a.H) &&
                            static_cast<uint32_t>(wi) < static_cast<uint32_t>(a.W);
            off[e] = in ? static_cast<uint32_t>((((n * a.H + hi) * a.W + wi) * a.C + T.c) * ES)
                        : kOutOfRange;
          }
        }
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_readfirstlane(T.isdy) ? dr : xr;
#pragma unroll
        for (int e = 0; e < E; ++e) R[i][e] = __builtin_amdgcn_raw_buffer_load_b128(rs, off[e], 0, 0);
      } else {
        // Element by element: column j of the chunk is channel / column
        // col + j, each with its own bounds (and tap for the patch).
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int m = m0 + e;
          union {
            i32x4 v;
            uint16_t h[8];
            float f[4];
          } u;
          u.v = i32x4{0, 0, 0, 0};
          if (T.on && m < m_end) {
#pragma unroll
            for (int j = 0; j < E; ++j) {
              const int col = T.col + j;
              int64_t idx = -1;
              if (T.isdy) {
                if (col < a.K) idx = static_cast<int64_t>(m) * a.K + col;
              } else if (col < a.Kg) {
                const int rs = col / a.C;
                const int r = rs / a.S;
                idx = patch_elem(m, r - a.pt, rs - r * a.S - a.pl, col - rs * a.C);
              }
              if (idx >= 0) {
                if constexpr (DT == FCONV_BF16)
                  u.h[j] = (T.isdy ? static_cast<const uint16_t*>(a.dy)
                                   : static_cast<const uint16_t*>(a.x))[idx];
                else
                  u.f[j] = (T.isdy ? static_cast<const float*>(a.dy)
                                   : static_cast<const float*>(a.x))[idx];
              }
            }
          }
          R[i][e] = u.v;
        }
      }
    }
  };

  auto stash = [&](int buf, const Task (&tasks)[TPT], const i32x4 (&R)[TPT][E]) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const Task& T = tasks[i];
      if (!T.on) continue;
      uint8_t* base = lds + buf * STAGE_BYTES;
      // Opaque copy: keeps the compiler from hoisting the E row addresses
      // of every task and buffer out of the stage loop (they would not fit
      // in registers); each costs one xor per stage here.
      int la = T.laddr;
      asm volatile("" : "+v"(la));
#pragma unroll
      for (int j = 0; j < E; ++j) {
        // Channel j of the chunk for the E pixels: the transposed block's
        // row j (pixel e at element e).
        i32x4 o;
        if constexpr (DT == FCONV_BF16) {
          const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
          for (int d = 0; d < 4; ++d)
            o[d] = static_cast<int32_t>(__builtin_amdgcn_perm(
                static_cast<uint32_t>(R[i][2 * d + 1][j >> 1]),
                static_cast<uint32_t>(R[i][2 * d][j >> 1]), sel));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = R[i][e][j];
        }
        *reinterpret_cast<i32x4*>(base + j * kWgRowBytes + (la ^ (j << 4))) = o;
      }
    }
  };

  f32x4 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Fragment addresses (stage-relative) of k-step 0, fixed for the whole
  // loop: row r reads pixel group g at slot g ^ f(r).  K-step 1 reads group
  // 4 + g, whose slot differs in bit 2: the address xor 64.
  const int g = lane >> 4;
  int aaddr[NI], baddr[NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = wk * 64 + 16 * i + (lane & 15);
    aaddr[i] = row * kWgRowBytes + wg_slot(row, g) * 16;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int row = TK + wkk * (NJ * 16) + 16 * j + (lane & 15);
    baddr[j] = row * kWgRowBytes + wg_slot(row, g) * 16;
  }

  auto compute = [&](int buf) {
    const uint8_t* base = lds + buf * STAGE_BYTES;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      i32x4 bfr[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        bfr[j] = *reinterpret_cast<const i32x4*>(base + (baddr[j] ^ (q << 6)));
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const i32x4 af = *reinterpret_cast<const i32x4*>(base + (aaddr[i] ^ (q << 6)));
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = wg_mma<DT>(af, bfr[j], acc[i][j]);
      }
    }
  };

  // Even stages use role 0, register set R0 and LDS buffer 0; odd stages
  // role 1, R1 and buffer 1.  Stage st's registers are refilled with stage
  // st + 2 right after they are written to LDS.
  i32x4 R0[TPT][E], R1[TPT][E];
  if (nst > 0) fetch(0, tk[0], R0);
  if (nst > 1) fetch(1, tk[1], R1);
  for (int st = 0; st < nst; st += 2) {
    stash(0, tk[0], R0);
    if (st + 2 < nst) fetch(st + 2, tk[0], R0);
    __syncthreads();
    compute(0);
    if (st + 1 >= nst) break;
    stash(1, tk[1], R1);
    if (st + 3 < nst) fetch(st + 3, tk[1], R1);
    __syncthreads();
    compute(1);
  }

  wg_store<NI, NJ>(a, acc, split, k0, kk0, wk, wkk, lane);
}

// ------------------------------------------------ direct-to-LDS kernel
//
// For C and K multiples of the 16-byte chunk.  Both operands are copied into
// LDS in their natural, pixel-major layout by buffer->LDS copies (no
// registers, no transposes): a stage holds BM pixel rows of dy (TK channels)
// followed by BM pixel rows of the patch matrix (128 columns).  Each 16-byte
// slot s of pixel row p is stored at slot s ^ swz(p).
//
// Fragments.  bf16: the gfx950 transposed LDS read (ds_read_b64_tr_b16)
// works on 16-lane groups: lane i's element e is element i % 4 of the
// 64-bit chunk addressed by lane 4e + i / 4 of its group (measured on the
// device).  Lane (j, g) (j = lane % 16, g = lane / 16) therefore addresses
// pixel row 8g + 4h + j / 4, columns c0 + 4 (j % 4) .. +3, and receives column
// c0 + j at pixels 8g + 4h .. +3: two reads (h = 0, 1) give the 8-pixel
// MFMA fragment of column c0 + j, for both operands alike.  fp32: one
// element per lane per 16x16x4 MFMA, read as is (pixel 4 kstep + g,
// column c0 + j).
//
// Swizzles.  bf16: one transposed read touches pixel rows 8g + 4h + (0..3)
// of the 4 groups, 32 bytes each; swz(p) = 2 (p & 3) + 8 ((p >> 3) & 1) puts
// them on 8 distinct 32-byte bank groups, twice over, the minimum for 512
// bytes.  fp32: a read touches 4 rows, 64 bytes each; swz(p) = 4 (p & 3)
// separates them.
//
// Pipeline (as the forward tiled kernel): NBUF LDS stage buffers (4, or 8
// for fp32 at one workgroup per CU), each its own __shared__ array; copies
// run NBUF - 1 stages ahead; a step waits for its own copies of the stage,
// meets the other waves at a plain barrier, issues the copies NBUF - 1
// stages ahead into the buffer of the stage before, reads the stage's
// fragments and runs its MFMAs.
template <int DT, int TK>
struct DmaCfg {
  static constexpr int ES = DT == FCONV_BF16 ? 2 : 4;
  static constexpr int BM = DT == FCONV_BF16 ? 32 : 16;  // pixels per stage
  static constexpr int RB_DY = TK * ES;                  // bytes per dy row
  static constexpr int RB_P = kWgTKK * ES;               // bytes per patch row
  static constexpr int DY_BYTES = BM * RB_DY;
  static constexpr int SB = DY_BYTES + BM * RB_P;        // stage bytes
  static constexpr int NW = TK == 256 ? 8 : 4;           // waves: 64x64 (or 64x32) each
  static constexpr int NC = SB / 1024;                   // 1 KiB copies per stage
  static constexpr int NCW = NC / NW;                    // per wave
  static_assert(SB % (NW * 1024) == 0, "stage must split into whole 1 KiB copies per wave");
  static_assert(DY_BYTES % 1024 == 0, "dy rows must fill whole copies");
};

// Slot xor of pixel row p in a row of RB bytes (RB / 16 slots; the xor
// stays inside the row).  A bf16 transposed read serves half a wave at a
// time: lane groups 0 and 1, each reading a 32-byte run of 4 consecutive
// pixel rows, the second group's rows 8 further on.  Bits 0-1 of p spread a
// group's four runs over distinct slot pairs; bit 3 of p puts the two groups
// on different banks: by flipping slot bit 3 in rows of 256 bytes or more,
// and slot bit 1 in 128-byte rows (where rows p and p + 8 sit on the same 32
// banks).  Measured: 1.3 conflict cycles per LDS instruction in the
// 64-channel tile without the 128-byte-row term.
template <int DT, int RB>
__device__ inline int dma_swz(int p) {
  if constexpr (DT == FCONV_BF16) {
    if constexpr (RB == 128) return ((2 * (p & 3)) ^ (((p >> 3) & 1) << 1)) & 7;
    return (((p & 3) << 1) | (((p >> 3) & 1) << 3)) & (RB / 16 - 1);
  }
  return ((p & 3) << 2) & (RB / 16 - 1);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_t;
typedef __attribute__((address_space(3))) float* lds_f32_t;

// s_waitcnt immediate for vmcnt(n) alone (gfx9: vmcnt bits [3:0] and
// [15:14]; expcnt and lgkmcnt at their maximum, i.e. not waited on).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// KS = 2: two groups of NW waves, each with its own LDS ring, split the
// workgroup's pixel range in two halves (group 0 the first, whole stages),
// and group 1's tile is added to group 0's through LDS at the end.  A
// workgroup then covers twice the pixels with the same waves per CU, so the
// ranges, and the partial tiles written and summed, are halved.
template <int DT, int TK, int NBUF, int KS>
__global__ __launch_bounds__((TK == 256 ? 512 : 256) * KS)  // DmaCfg::NW waves per group
__attribute__((amdgpu_waves_per_eu(NBUF == 8 ? 1 : 2, 2)))  // the 8-stage ring fills a CU's LDS
void wgrad_dma_kernel(WgArgs a) {
  using Cfg = DmaCfg<DT, TK>;
  constexpr int ES = Cfg::ES, BM = Cfg::BM, NCW = Cfg::NCW, NW = Cfg::NW;
  static_assert(KS == 1 || (KS == 2 && NW == 4 && NBUF == 4), "two groups of four waves, 4-stage rings");
  constexpr int E = 16 / ES;
  constexpr int WK = TK / 64;
  constexpr int WKK = NW / WK;
  constexpr int NI = 4;
  constexpr int NJ = kWgTKK / WKK / 16;
  static_assert(NBUF == 4 || NBUF == 8, "ring of 4 or 8 stages");
  constexpr int SB_HI = NBUF > 4 ? Cfg::SB : 16;
  // Stage buffer i of group q at bufi + q * SB.
  __shared__ __attribute__((aligned(1024))) char buf0[KS * Cfg::SB];
  __shared__ __attribute__((aligned(1024))) char buf1[KS * Cfg::SB];
  __shared__ __attribute__((aligned(1024))) char buf2[KS * Cfg::SB];
  __shared__ __attribute__((aligned(1024))) char buf3[KS * Cfg::SB];
  __shared__ __attribute__((aligned(1024))) char buf4[SB_HI];
  __shared__ __attribute__((aligned(1024))) char buf5[SB_HI];
  __shared__ __attribute__((aligned(1024))) char buf6[SB_HI];
  __shared__ __attribute__((aligned(1024))) char buf7[SB_HI];

  const int nb = gridDim.x;
  const int b = blockIdx.x;
  const int logical = (nb % 8 == 0) ? (b % 8) * (nb / 8) + b / 8 : b;
  if (logical >= a.blocks) return;
  const int tiles = a.tiles_k * a.tiles_kk;
  const int split = logical / tiles;
  const int tile = logical % tiles;
  const int k0 = (tile % a.tiles_k) * TK;
  const int kk0 = (tile / a.tiles_k) * kWgTKK;
  const int r_begin = split * a.m_per_split;
  const int r_end = min(a.M, r_begin + a.m_per_split);
  const int r_st = (r_end - r_begin + BM - 1) / BM;  // stages of the range

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave0 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave0 / NW;      // wave group (KS = 2), else 0
  const int wave = wave0 % NW;     // wave inside the group
  const int wk = wave % WK, wkk = wave / WK;
  // The group's pixels [m_begin, m_end) and the stages every group steps
  // through (group 1's past its pixels copy zeros).
  const int nst = (r_st + KS - 1) / KS;
  const int m_begin = r_begin + grp * nst * BM;
  const int m_end = min(r_end, m_begin + nst * BM);
  char* const bufs[8] = {buf0 + grp * Cfg::SB, buf1 + grp * Cfg::SB, buf2 + grp * Cfg::SB,
                         buf3 + grp * Cfg::SB, buf4, buf5, buf6, buf7};

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t dr = make_rsrc(a.dy, a.dy_bytes);

  // This wave's copies: q = wave + NW i.  Lane l of copy q fills stage bytes
  // q * 1024 + 16 l: pixel row p and stored slot s' there, i.e. the chunk
  // s = s' ^ swz(p) of that row.
  int c_p[NCW], c_col[NCW], c_dr[NCW], c_ds[NCW], c_c[NCW];
  bool c_ok[NCW];
#pragma unroll
  for (int i = 0; i < NCW; ++i) {
    const int q = wave + NW * i;
    const int byte = q * 1024 + lane * 16;
    const bool isdy = q * 1024 < Cfg::DY_BYTES;  // wave-uniform
    const int rb = isdy ? Cfg::RB_DY : Cfg::RB_P;
    const int rel = isdy ? byte : byte - Cfg::DY_BYTES;
    const int p = rel / rb;
    const int s = ((rel % rb) / 16) ^ (isdy ? dma_swz<DT, Cfg::RB_DY>(p) : dma_swz<DT, Cfg::RB_P>(p));
    c_p[i] = p;
    c_col[i] = (isdy ? k0 : kk0) + s * E;
    c_dr[i] = c_ds[i] = c_c[i] = 0;
    if (isdy) {
      c_ok[i] = c_col[i] < a.K;
    } else {
      c_ok[i] = c_col[i] < a.Kg;
      const int rs = c_col[i] / a.C;
      c_c[i] = c_col[i] - rs * a.C;
      const int r = rs / a.S;
      c_dr[i] = r - a.pt;
      c_ds[i] = rs - r * a.S - a.pl;
    }
  }

  int nx_st = 0;
  auto issue = [&](char* buf) __attribute__((always_inline)) {
    const int st = nx_st++;
    const int mb = m_begin + st * BM;
#pragma unroll
    for (int i = 0; i < NCW; ++i) {
      const int q = wave + NW * i;
      const int m = mb + c_p[i];
      const bool live = c_ok[i] && st < nst && m < m_end;
      uint32_t off = kOutOfRange;
      if (q * 1024 < Cfg::DY_BYTES) {
        if (live) off = static_cast<uint32_t>((m * a.K + c_col[i]) * ES);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(dr, (lds_ptr_t)(buf + q * 1024), 16, off, 0, 0, 0);
      } else {
        const uint32_t um = static_cast<uint32_t>(live ? m : 0);
        const uint32_t n = fast_div(um, a.hw_mul, a.hw_add, a.hw_shift);
        const uint32_t rem = um - n * static_cast<uint32_t>(a.Ho * a.Wo);
        const uint32_t ho = fast_div(rem, a.wo_mul, a.wo_add, a.wo_shift);
        const int wo = static_cast<int>(rem - ho * static_cast<uint32_t>(a.Wo));
        const int hi = static_cast<int>(ho) * a.sh + c_dr[i];
        const int wi = wo * a.sw + c_ds[i];
        if (live && static_cast<uint32_t>(hi) < static_cast<uint32_t>(a.H) &&
            static_cast<uint32_t>(wi) < static_cast<uint32_t>(a.W))
          off = static_cast<uint32_t>(
              (((static_cast<int>(n) * a.H + hi) * a.W + wi) * a.C + c_c[i]) * ES);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(buf + q * 1024), 16, off, 0, 0, 0);
      }
    }
  };

  f32x4 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int j16 = lane & 15, g = lane >> 4;
  // Fragment addresses, stage-relative.
  constexpr int NH = DT == FCONV_BF16 ? 2 : 4;  // bf16: two tr reads; fp32: 4 k-steps
  int aaddr[NH][NI], baddr[NH][NJ];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int col = wk * 64 + 16 * i;
      if constexpr (DT == FCONV_BF16) {
        const int p = 8 * g + 4 * h + (j16 >> 2);
        const int cb = (col + 4 * (j16 & 3)) * 2;  // byte in row
        aaddr[h][i] = p * Cfg::RB_DY + (((cb >> 4) ^ dma_swz<DT, Cfg::RB_DY>(p)) << 4) + (cb & 15);
      } else {
        const int p = 4 * h + g;
        const int cb = (col + j16) * 4;
        aaddr[h][i] = p * Cfg::RB_DY + (((cb >> 4) ^ dma_swz<DT, Cfg::RB_DY>(p)) << 4) + (cb & 15);
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = wkk * (NJ * 16) + 16 * j;
      if constexpr (DT == FCONV_BF16) {
        const int p = 8 * g + 4 * h + (j16 >> 2);
        const int cb = (col + 4 * (j16 & 3)) * 2;
        baddr[h][j] = Cfg::DY_BYTES + p * Cfg::RB_P + (((cb >> 4) ^ dma_swz<DT, Cfg::RB_P>(p)) << 4) + (cb & 15);
      } else {
        const int p = 4 * h + g;
        const int cb = (col + j16) * 4;
        baddr[h][j] = Cfg::DY_BYTES + p * Cfg::RB_P + (((cb >> 4) ^ dma_swz<DT, Cfg::RB_P>(p)) << 4) + (cb & 15);
      }
    }
  }

  auto mma_stage = [&](const char* buf) __attribute__((always_inline)) {
    if constexpr (DT == FCONV_BF16) {
      v4i16 al[NI][2], bl[NJ][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
          al[i][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)(buf + aaddr[h][i]));
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          bl[j][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)(buf + baddr[h][j]));
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const bf16x8 af = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(al[i][0], al[i][1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const bf16x8 bf = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(bl[j][0], bl[j][1], 0, 1, 2, 3, 4, 5, 6, 7));
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[i][j], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        float al[NI], bl[NJ];
#pragma unroll
        for (int i = 0; i < NI; ++i) al[i] = *(lds_f32_t)(buf + aaddr[h][i]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) bl[j] = *(lds_f32_t)(buf + baddr[h][j]);
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(al[i], bl[j], acc[i][j], 0, 0, 0);
      }
    }
  };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  int st = 0;
  // Stage st lives in buffer st % NBUF.  Two stages per barrier (3-6%
  // faster than one on the bf16 layers, 1% on fp32): this wave's copies of
  // stages st and st + 1 have landed before it (those of the NBUF - 4 later
  // stages may still be in flight), then stages st + NBUF - 2 and
  // st + NBUF - 1 are copied into the buffers of st - 2 and st - 1
  // (consumed by the previous double step's MFMAs).
  auto dwait = [&]() __attribute__((always_inline)) {
    constexpr int imm = vmcnt_imm((NBUF - 4) * NCW);
    __builtin_amdgcn_s_waitcnt(imm);
  };
  auto dstep = [&](const char* c0, const char* c1, char* f0, char* f1)
      __attribute__((always_inline)) {
    dwait();
    barrier();
    issue(f0);
    issue(f1);
    mma_stage(c0);
    mma_stage(c1);
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int i = 0; i < NBUF - 2; ++i) issue(bufs[i]);
  for (; st + NBUF <= nst; st += NBUF) {
#pragma unroll
    for (int i = 0; i < NBUF; i += 2)
      dstep(bufs[i], bufs[i + 1], bufs[(i + NBUF - 2) % NBUF], bufs[(i + NBUF - 1) % NBUF]);
  }
  // The rest: whole double steps, then a last single stage.
#pragma unroll
  for (int i = 0; i < NBUF - 2; i += 2)
    if (st + i + 2 <= nst)
      dstep(bufs[i], bufs[i + 1], bufs[(i + NBUF - 2) % NBUF], bufs[(i + NBUF - 1) % NBUF]);
  const int rest = (nst - st) & ~1;  // stages done by the double steps above
  if (st + rest < nst) {
    __builtin_amdgcn_s_waitcnt(0);
    barrier();
#pragma unroll
    for (int i = 0; i < NBUF; i += 2)
      if (i == rest) mma_stage(bufs[i]);
  }
  __builtin_amdgcn_s_waitcnt(0);  // copies past the last stage (zeros) land before exit

  if constexpr (KS == 2) {
    // Group 1 hands its tile to group 0 through the stage buffers (every
    // wave has read its last stage before the barrier): piece t = i*NJ + j
    // of wave w at buffer t % 4, offset (w * NI*NJ/4 + t/4) KiB.
    static_assert(NW * (NI * NJ / 4) * 1024 <= KS * Cfg::SB, "hand-off fits the stage buffers");
    char* const hb[4] = {buf0, buf1, buf2, buf3};
    barrier();
    if (grp == 1) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int t = i * NJ + j;
          *reinterpret_cast<f32x4*>(hb[t % 4] + (wave * (NI * NJ / 4) + t / 4) * 1024 + 16 * lane) =
              acc[i][j];
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the hand-off is written
    barrier();
    if (grp == 1) return;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int t = i * NJ + j;
        acc[i][j] += *reinterpret_cast<const f32x4*>(
            hb[t % 4] + (wave * (NI * NJ / 4) + t / 4) * 1024 + 16 * lane);
      }
  }
  wg_store<NI, NJ>(a, acc, split, k0, kk0, wk, wkk, lane);
}

// Row-halo weight gradient (bf16, 3x3, stride 1): the direct-to-LDS kernel
// copies, for every 128-column tile, the patch rows of its two or three taps,
// so each input pixel crosses from L2 into LDS once per tap tile and each
// gradient pixel once per tile.  Here a workgroup owns 9 taps x 32 input
// channels x 64 output channels of dw over a range of output rows, and every
// input row and gradient row of the range is copied into LDS once: the taps
// are LDS address offsets.
//
// Waves 0-3 (one per SIMD) run the MFMAs; wave m holds the 9 taps x 16
// channels (channel tile m>>1 of the 32) x 32 output channels (tiles
// 2(m&1), 2(m&1)+1 of the 64): 18 accumulator tiles.  Waves 4-7 issue every
// copy: their code holds no LDS reads that a pending copy could alias, and
// the MFMA waves' code no copies, so the compiler adds no memory-count wait to
// either.  A step is one output row (Wo > 32: two 32-pixel blocks of the row)
// or two output rows (Wo <= 32: one block each); per block a wave reads two
// dy fragments and nine patch fragments (gfx950's transposed LDS read, as in
// the direct-to-LDS kernel) and runs 18 MFMAs.
//
// Input rows live in a ring of twelve 64-pixel slots (32 channels, 4 KiB):
// rows are numbered in the order the workgroup's output rows first need them
// (row r of output row u is number k0(u) + r; k0 advances by 1 per output row
// and by 3 at an image change), number k in slot k % 12.  The rows of the
// three steps in flight span at most twelve numbers: 5 + 2 per image change
// for one-row steps (at most two changes in three rows), 8 + 2 per change for
// two-row steps (at most two changes in six rows when Ho >= 3).  Pixel place X (= input
// column + left pad) holds its four 16-byte chunks at X*64 + 16*(c ^ 2((X>>3)&1)).
// Gradient rows: a ring of three 8 KiB slots, one per step (64 pixel places
// of 64 channels, the direct-to-LDS kernel's swizzle).  In the interval that
// ends with the barrier after MFMA step t, the copy waves copy step t+2's
// new input rows and gradient rows, then wait for step t+1's (issued one
// interval earlier): the MFMA waves read only rows published by a barrier.
constexpr int kWhThreads = 512;
constexpr int kWhXSlots = 12;
constexpr int kWhXSlot = 4096;   // 64 pixel places x 32 channels x 2 bytes
constexpr int kWhDySlots = 3;
constexpr int kWhDySlot = 8192;  // 64 pixel places x 64 channels x 2 bytes

// Row number of row 0 of output row gr (flattened n*Ho + ho) for a workgroup
// that starts at output row ho0 of image n0.
__device__ inline int wh_k0(const WgArgs& a, int gr, int n0, int ho0) {
  const int n = static_cast<int>(fast_div(static_cast<uint32_t>(gr), a.ho_mul, a.ho_add, a.ho_shift));
  const int ho = gr - n * a.Ho;
  if (n == n0) return ho - ho0;
  return a.Ho + 2 - ho0 + (n - n0 - 1) * (a.Ho + 2) + ho;
}

// Slot xor of input pixel place X (64-byte rows, 4 slots): a transposed
// read's two lane groups per half wave read places 8 apart, which share
// banks unless bit 3 of X flips slot bit 1 (a 32-byte run is a slot pair).
__device__ inline int wh_xswz(int X) { return ((X >> 3) & 1) << 1; }

template <int RPS>
__global__ __launch_bounds__(kWhThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void wgrad_halo_kernel(WgArgs a) {
  using Cfg = DmaCfg<FCONV_BF16, 64>;  // the 128-byte gradient rows' swizzle
  __shared__ __attribute__((aligned(1024))) char xring[kWhXSlots * kWhXSlot];
  __shared__ __attribute__((aligned(1024))) char dring[kWhDySlots * kWhDySlot];

  const int nb = gridDim.x;
  const int bidx = blockIdx.x;
  const int logical = (nb % 8 == 0) ? (bidx % 8) * (nb / 8) + bidx / 8 : bidx;
  if (logical >= a.blocks) return;  // uniform per workgroup
  const int tiles = a.tiles_k * a.tiles_kk;
  const int split = logical / tiles;
  const int tile = logical % tiles;
  const int kb = tile % a.tiles_k;   // 64-channel block of K
  const int cs = tile / a.tiles_k;   // 32-channel slice of C
  const int rows_total = a.N * a.Ho;
  const int g0 = split * a.m_per_split;  // first output row
  const int nrows = min(g0 + a.m_per_split, rows_total) - g0;
  const int steps = (nrows + RPS - 1) / RPS;
  const int n0 = static_cast<int>(fast_div(static_cast<uint32_t>(g0), a.ho_mul, a.ho_add, a.ho_shift));
  const int ho0 = g0 - n0 * a.Ho;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  if (wave < 4) {
    const int ct = wave >> 1, kp = wave & 1;
    const int j16 = lane & 15, g = lane >> 4;
    // Fragment offsets: gradient, inside a block (pixel place p of its
    // first); input, inside a row slot for block bb (place 32bb + p + s for
    // Wo > 32, else p + s; places past 63 belong to pixels past Wo, whose
    // gradient is zero, and read place 63 instead, inside the slot).
    int dyo[2][2], xo[2][2][3];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int p = 8 * g + 4 * h + (j16 >> 2);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int cb = ((2 * kp + kt) * 16 + 4 * (j16 & 3)) * 2;
        dyo[h][kt] = p * Cfg::RB_DY + (((cb >> 4) ^ dma_swz<FCONV_BF16, Cfg::RB_DY>(p)) << 4) + (cb & 15);
      }
      const int cbx = (ct * 16 + 4 * (j16 & 3)) * 2;
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int s = 0; s < 3; ++s) {
          const int X = min((RPS == 1 ? 32 * bb : 0) + p + s, 63);
          xo[bb][h][s] = X * 64 + (((cbx >> 4) ^ wh_xswz(X)) << 4) + (cbx & 15);
        }
    }
    f32x4 acc[9][2];
#pragma unroll
    for (int q = 0; q < 9; ++q)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) acc[q][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    barrier();  // steps 0 and 1 have landed
    for (int t = 0; t < steps; ++t) {
      const char* dbase = dring + (t % kWhDySlots) * kWhDySlot;
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        // Block bb: pixels 32bb.. of output row RPS*t (RPS = 1), or output
        // row RPS*t + bb (RPS = 2); rows past the range are skipped.
        const int u = RPS * t + (RPS == 2 ? bb : 0);
        if (u >= nrows) continue;  // uniform
        const int k0 = wh_k0(a, g0 + u, n0, ho0);
        const int pix0 = RPS == 1 ? 32 * bb : 0;
        const char* db = dbase + (RPS == 2 ? bb * 4096 : 0) + pix0 * Cfg::RB_DY;
        v4i16 al[2][2], bl[9][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
            al[kt][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)(db + dyo[h][kt]));
#pragma unroll
          for (int r = 0; r < 3; ++r) {
            const char* xb = xring + ((k0 + r) % kWhXSlots) * kWhXSlot;
#pragma unroll
            for (int s = 0; s < 3; ++s)
              bl[3 * r + s][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)(xb + xo[bb][h][s]));
          }
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const bf16x8 af = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(al[kt][0], al[kt][1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int q = 0; q < 9; ++q) {
            const bf16x8 bf = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(bl[q][0], bl[q][1], 0, 1, 2, 3, 4, 5, 6, 7));
            acc[q][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[q][kt], 0, 0, 0);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this step's reads are done
      barrier();
    }
    // The tile: lane holds D[k][kk] for k = 64 kb + 16 (2 kp + kt) + 4 g + 0..3
    // and kk = (r, s, c) with c = 32 cs + 16 ct + j16.
    const bool kvec4 = (a.K & 3) == 0;
#pragma unroll
    for (int q = 0; q < 9; ++q)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int k = kb * 64 + (2 * kp + kt) * 16 + 4 * g;
        const int kk = q * a.C + cs * 32 + ct * 16 + j16;
        const f32x4 v = acc[q][kt];
        const int64_t base = static_cast<int64_t>(kk) * a.K + k;
        if (a.out_mode == 0) {
          float* o = static_cast<float*>(a.out) + split * a.lp + base;
          if (kvec4) *reinterpret_cast<f32x4*>(o) = v;
          else for (int t4 = 0; t4 < 4; ++t4) o[t4] = v[t4];
        } else if (a.out_mode == 1) {
          float* o = static_cast<float*>(a.out) + base;
          if (kvec4) *reinterpret_cast<f32x4*>(o) = v;
          else for (int t4 = 0; t4 < 4; ++t4) o[t4] = v[t4];
        } else {
          uint16_t* o = static_cast<uint16_t*>(a.out) + base;
          const uint32_t lo = f32_to_bf16_rne(v[0]) | (uint32_t(f32_to_bf16_rne(v[1])) << 16);
          const uint32_t hi = f32_to_bf16_rne(v[2]) | (uint32_t(f32_to_bf16_rne(v[3])) << 16);
          *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
        }
      }
  } else {
    const int e = wave - 4;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(a.dy, a.dy_bytes);
    // This wave copies KiB e of every input row: per lane the source offset
    // inside the row (out-of-range columns: 2^31, which keeps the sum with any
    // row's offset, below 2^31, out of range), and KiBs e and e + 4 of every
    // gradient slot.
    uint32_t xoff;
    {
      const int pos = e * 1024 + lane * 16;
      const int X = pos / 64;
      const int c = ((pos % 64) >> 4) ^ wh_xswz(X);
      const int wi = X - a.pl;
      xoff = static_cast<unsigned>(wi) < static_cast<unsigned>(a.W)
                 ? static_cast<uint32_t>((wi * a.C + cs * 32 + c * 8) * 2)
                 : kOutOfRange;
    }
    int dpx[2], dch[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pos = (e + 4 * i) * 1024 + lane * 16;
      const int p = pos / Cfg::RB_DY;  // pixel place in the 64-place slot
      dpx[i] = p;
      dch[i] = kb * 64 + (((pos % Cfg::RB_DY) >> 4) ^ dma_swz<FCONV_BF16, Cfg::RB_DY>(p)) * 8;
    }
    // Step u's new input rows and its gradient rows; returns the copies issued.
    auto copy_step = [&](int u) -> int {
      if (u >= steps) return 0;
      int issued = 0;
#pragma unroll
      for (int b = 0; b < RPS; ++b) {
        const int ur = RPS * u + b;
        if (ur >= nrows) break;
        const int gr = g0 + ur;
        const int n = static_cast<int>(fast_div(static_cast<uint32_t>(gr), a.ho_mul, a.ho_add, a.ho_shift));
        const int ho = gr - n * a.Ho;
        const int k0 = wh_k0(a, gr, n0, ho0);
        // Rows 0 and 1 of output row ur are rows 1 and 2 of the previous one
        // unless ur starts the range or an image.
        for (int r = (ur == 0 || ho == 0) ? 0 : 2; r < 3; ++r) {
          const int hi = ho - a.pt + r;
          const bool ok = static_cast<unsigned>(hi) < static_cast<unsigned>(a.H);
          const uint32_t rbase = static_cast<uint32_t>((n * a.H + hi) * a.W * a.C * 2);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              xr, (lds_ptr_t)(xring + ((k0 + r) % kWhXSlots) * kWhXSlot + e * 1024), 16,
              ok ? rbase + xoff : kOutOfRange, 0, 0, 0);
          ++issued;
        }
      }
      char* ds = dring + (u % kWhDySlots) * kWhDySlot;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        // RPS = 1: places 0..63 of row u; RPS = 2: places 32b + wo of row 2u + b.
        const int b = RPS == 2 ? dpx[i] >> 5 : 0;
        const int wo = RPS == 2 ? dpx[i] & 31 : dpx[i];
        const int ur = RPS * u + b;
        const bool ok = ur < nrows && wo < a.Wo;
        const uint32_t src =
            ok ? static_cast<uint32_t>(((static_cast<int64_t>(g0 + ur) * a.Wo + wo) * a.K + dch[i]) * 2)
               : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(dr, (lds_ptr_t)(ds + (e + 4 * i) * 1024), 16, src,
                                                 0, 0, 0);
        ++issued;
      }
      return issued;
    };
    copy_step(0);
    copy_step(1);
    // Steps 0 and 1: the MFMA waves read only rows published by a barrier.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    barrier();
    for (int t = 0; t < steps; ++t) {
      const int c = copy_step(t + 2);
      // Step t+1's copies (issued one interval earlier) have landed; this
      // interval's may stay in flight.
      switch (c) {
#define FCONV_WH_WAIT(n) \
  case n:                \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(n)); \
    break;
        FCONV_WH_WAIT(0) FCONV_WH_WAIT(1) FCONV_WH_WAIT(2) FCONV_WH_WAIT(3) FCONV_WH_WAIT(4)
        FCONV_WH_WAIT(5) FCONV_WH_WAIT(6) FCONV_WH_WAIT(7) FCONV_WH_WAIT(8)
#undef FCONV_WH_WAIT
        default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
      }
      barrier();
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
}

// dw[i] = sum over pixel ranges z of part[z][i], in a fixed association
// (zeros for no range).  A workgroup of 256 threads owns 256/G four-element
// columns; its G lane groups each add the ranges z = g, g + G, g + 2G, ... in
// increasing order, with up to four of those loads in flight together, and
// the G group sums are then added in group order.  Many ranges are thus read
// in parallel (the sum is bound by the partials' bandwidth, not by the
// latency of one long chain), and every run of a plan adds the same values in
// the same order.  G = 4 for up to 8 ranges (a quarter of the workgroups that
// 16 groups would need, most of whose threads would have no range to read),
// else 16.
template <int G>
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const float* __restrict__ part,
                                                           void* __restrict__ dw, int splits,
                                                           int64_t lp, int64_t L, int out_bf16) {
  constexpr int COLS = 256 / G;
  __shared__ f32x4 red[G][COLS];
  const int col = threadIdx.x % COLS;
  const int g = threadIdx.x / COLS;
  const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * COLS + col) * 4;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if (i0 < L) {
    for (int z0 = g; z0 < splits; z0 += 4 * G) {
      f32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int z = z0 + u * G;
        v[u] = z < splits ? *reinterpret_cast<const f32x4*>(part + z * lp + i0)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (z0 + u * G < splits) s += v[u];
    }
  }
  red[g][col] = s;
  __syncthreads();
  if (g != 0 || i0 >= L) return;
  s = red[0][col];
#pragma unroll
  for (int q = 1; q < G; ++q) s += red[q][col];
  if (out_bf16) {
    uint16_t* o = static_cast<uint16_t*>(dw) + i0;
    if (i0 + 4 <= L && (L & 3) == 0) {
      const uint32_t lo = f32_to_bf16_rne(s[0]) | (uint32_t(f32_to_bf16_rne(s[1])) << 16);
      const uint32_t hi = f32_to_bf16_rne(s[2]) | (uint32_t(f32_to_bf16_rne(s[3])) << 16);
      *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
    } else {
      for (int t = 0; t < 4 && i0 + t < L; ++t) o[t] = f32_to_bf16_rne(s[t]);
    }
  } else {
    float* o = static_cast<float*>(dw) + i0;
    if (i0 + 4 <= L && (L & 3) == 0) {
      *reinterpret_cast<f32x4*>(o) = s;
    } else {
      for (int t = 0; t < 4 && i0 + t < L; ++t) o[t] = s[t];
    }
  }
}

// The sum of the ranges (splits = 0: zeros) with the lane groups chosen by
// the number of ranges.
hipError_t launch_wgrad_reduce(const float* part, void* dw, int splits, int64_t lp, int64_t L,
                               int out_bf16, hipStream_t s) {
  if (splits <= 8) {
    const int grid = static_cast<int>((L + 4 * 64 - 1) / (4 * 64));
    hipLaunchKernelGGL(wgrad_reduce_kernel<4>, dim3(grid), dim3(256), 0, s, part, dw, splits, lp,
                       L, out_bf16);
  } else {
    const int grid = static_cast<int>((L + 4 * 16 - 1) / (4 * 16));
    hipLaunchKernelGGL(wgrad_reduce_kernel<16>, dim3(grid), dim3(256), 0, s, part, dw, splits,
                       lp, L, out_bf16);
  }
  return hipGetLastError();
}

template <int DT, int TK, bool VEC>
hipError_t launch_wgrad_main(const WgArgs& a, hipStream_t s) {
  const int grid = (a.blocks + 7) / 8 * 8;
  hipLaunchKernelGGL((wgrad_kernel<DT, TK, VEC>), dim3(grid), dim3(kWgThreads), 0, s, a);
  return hipGetLastError();
}

template <int DT, int TK, int NBUF, int KS = 1>
hipError_t launch_wgrad_dma(const WgArgs& a, hipStream_t s) {
  const int grid = (a.blocks + 7) / 8 * 8;
  hipLaunchKernelGGL((wgrad_dma_kernel<DT, TK, NBUF, KS>), dim3(grid),
                     dim3(DmaCfg<DT, TK>::NW * KS * 64), 0, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_wgrad_dt(const fconv_wgrad_plan_s* p, const WgArgs& a, hipStream_t s) {
  if constexpr (DT == FCONV_BF16) {
    if (p->halo) {
      const int grid = (a.blocks + 7) / 8 * 8;
      if (p->rps == 2)
        hipLaunchKernelGGL(wgrad_halo_kernel<2>, dim3(grid), dim3(kWhThreads), 0, s, a);
      else
        hipLaunchKernelGGL(wgrad_halo_kernel<1>, dim3(grid), dim3(kWhThreads), 0, s, a);
      return hipGetLastError();
    }
  }
  if (p->dma && p->tk == 256) return launch_wgrad_dma<DT, 256, 4>(a, s);
  if constexpr (DT == FCONV_BF16) {
    if (p->dma && p->ksplit)
      return p->tk == 128 ? launch_wgrad_dma<DT, 128, 4, 2>(a, s) : launch_wgrad_dma<DT, 64, 4, 2>(a, s);
  }
  if (p->dma)
    return p->ring == 8
               ? (p->tk == 128 ? launch_wgrad_dma<DT, 128, 8>(a, s) : launch_wgrad_dma<DT, 64, 8>(a, s))
               : (p->tk == 128 ? launch_wgrad_dma<DT, 128, 4>(a, s) : launch_wgrad_dma<DT, 64, 4>(a, s));
  if (p->tk == 128)
    return p->vec ? launch_wgrad_main<DT, 128, true>(a, s) : launch_wgrad_main<DT, 128, false>(a, s);
  return p->vec ? launch_wgrad_main<DT, 64, true>(a, s) : launch_wgrad_main<DT, 64, false>(a, s);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

const char* wgrad_kernel_name(int dtype, int tk, bool vec, bool dma, int ring, bool ksplit,
                              bool halo) {
  if (halo) return "wgrad_halo_bf16";
  if (dma && tk == 256) return "wgrad_dma_bf16_256";
  if (dma && ksplit) return tk == 128 ? "wgrad_dma2_bf16_128" : "wgrad_dma2_bf16_64";
  if (dma && ring == 8) {
    if (dtype == FCONV_BF16) return tk == 128 ? "wgrad_dma8_bf16_128" : "wgrad_dma8_bf16_64";
    return tk == 128 ? "wgrad_dma8_f32_128" : "wgrad_dma8_f32_64";
  }
  if (dma) {
    if (dtype == FCONV_BF16) return tk == 128 ? "wgrad_dma_bf16_128" : "wgrad_dma_bf16_64";
    return tk == 128 ? "wgrad_dma_f32_128" : "wgrad_dma_f32_64";
  }
  if (dtype == FCONV_BF16)
    return tk == 128 ? (vec ? "wgrad_bf16_128" : "wgrad_bf16_128_elem")
                     : (vec ? "wgrad_bf16_64" : "wgrad_bf16_64_elem");
  return tk == 128 ? (vec ? "wgrad_f32_128" : "wgrad_f32_128_elem")
                   : (vec ? "wgrad_f32_64" : "wgrad_f32_64_elem");
}

}  // namespace
}  // namespace fconv

extern "C" {

fconv_status fconv_wgrad_plan_create(const fconv_desc* desc, fconv_wgrad_plan* out) {
  using namespace fconv;
  if (!desc || !out) return FCONV_ERR_INVALID_ARG;
  *out = nullptr;
  const fconv_desc& d = *desc;
  if (d.dtype != FCONV_BF16 && d.dtype != FCONV_FP32) return FCONV_ERR_UNSUPPORTED;
  if (d.padding != FCONV_PAD_SAME && d.padding != FCONV_PAD_VALID) return FCONV_ERR_UNSUPPORTED;
  if (d.n_ops != 0 || (d.flags & ~FCONV_WGRAD_OUT_FP32)) return FCONV_ERR_UNSUPPORTED;
  if (d.N < 0 || d.H < 1 || d.W < 1 || d.C < 1 || d.K < 1 || d.R < 1 || d.S < 1 ||
      d.stride_h < 1 || d.stride_w < 1)
    return FCONV_ERR_INVALID_ARG;
  fconv_wgrad_plan_s* p = new (std::nothrow) fconv_wgrad_plan_s();
  if (!p) return FCONV_ERR_INVALID_ARG;
  p->d = d;
  const bool same = d.padding == FCONV_PAD_SAME;
  if (!resolve_axis(d.H, d.R, d.stride_h, same, &p->Ho, &p->pt, &p->pb) ||
      !resolve_axis(d.W, d.S, d.stride_w, same, &p->Wo, &p->pl, &p->pr)) {
    delete p;
    return FCONV_ERR_INVALID_ARG;
  }
  p->esize = d.dtype == FCONV_BF16 ? 2 : 4;
  p->E = 16 / p->esize;
  p->out_fp32 = d.dtype == FCONV_FP32 || (d.flags & FCONV_WGRAD_OUT_FP32) != 0;
  p->M = static_cast<int64_t>(d.N) * p->Ho * p->Wo;
  p->x_elems = static_cast<int64_t>(d.N) * d.H * d.W * d.C;
  p->dy_elems = p->M * d.K;
  const int64_t kg = static_cast<int64_t>(d.R) * d.S * d.C;
  p->dw_elems = kg * d.K;
  // Buffer descriptors and offsets are 32-bit.
  if (p->x_elems * p->esize >= INT32_MAX || p->dy_elems * p->esize >= INT32_MAX ||
      p->dw_elems >= INT32_MAX / 4 || p->M >= INT32_MAX) {
    delete p;
    return FCONV_ERR_UNSUPPORTED;
  }
  p->Kg = static_cast<int32_t>(kg);
  p->vec = d.C % p->E == 0 && d.K % p->E == 0;
  const int64_t bm = 8 * p->E;
  // FCONV_WGRAD_KERNEL=staged (environment) pins the register-staged
  // kernel on shapes the direct-to-LDS kernel takes; FCONV_WGRAD_RING=4|8
  // its LDS ring depth; FCONV_WGRAD_TK=128 the 128-channel tile where the
  // 256-channel one would be chosen (all for A/B comparisons).
  const char* force = getenv("FCONV_WGRAD_KERNEL");
  p->dma = p->vec && !(force && strcmp(force, "staged") == 0);
  // Ring depth: bf16 runs two workgroups per CU with 4-stage rings (the
  // second workgroup's MFMAs fill the first one's waits: 40.5 us against 57
  // with one 8-stage workgroup on the 28x28x256 layer); fp32, with 8x the
  // MFMA time per byte, one workgroup with an 8-stage ring (180 us against
  // 216).
  const char* ring = getenv("FCONV_WGRAD_RING");
  p->ring = d.dtype == FCONV_FP32 ? 8 : 4;
  if (ring && (atoi(ring) == 4 || atoi(ring) == 8)) p->ring = atoi(ring);
  // Tile width: 128 output channels, or 64 for K <= 64.  FCONV_WGRAD_TK=256
  // pins 256-channel tiles (eight waves of 64x64, one workgroup per CU, a
  // quarter fewer operand bytes per flop) for bf16 with K > 128 on the
  // 4-stage ring: as fast as two wave groups on 128-channel tiles on the
  // 28x28x256 layer, with twice their pixel ranges and partial sums.
  const char* tk_env = getenv("FCONV_WGRAD_TK");
  const bool wide = p->dma && d.dtype == FCONV_BF16 && p->ring == 4 && d.K > 128 && tk_env &&
                    atoi(tk_env) == 256;
  p->tk = wide ? 256 : d.K > 64 ? 128 : 64;
  // Two wave groups per workgroup splitting each pixel range (bf16, 4-stage
  // ring, 64/128-channel tiles): one workgroup of eight waves per CU instead
  // of two of four, half the ranges.  FCONV_WGRAD_GROUPS=1 pins one group.
  const char* groups = getenv("FCONV_WGRAD_GROUPS");
  p->ksplit = p->dma && d.dtype == FCONV_BF16 && p->ring == 4 && p->tk != 256 &&
              !(groups && atoi(groups) == 1);
  p->tiles_k = (d.K + p->tk - 1) / p->tk;
  p->tiles_kk = (p->Kg + kWgTKK - 1) / kWgTKK;
  const int64_t tiles = static_cast<int64_t>(p->tiles_k) * p->tiles_kk;
  // Pixel ranges, each at least four stages long per wave group: one
  // workgroup per CU with the 8-stage ring, the 256-channel tile or two wave
  // groups, else about two per CU.
  const bool one_per_cu = p->dma && (p->ring == 8 || p->tk == 256 || p->ksplit);
  int64_t splits = one_per_cu ? kWgTargetBlocks / 2 / tiles
                              : (kWgTargetBlocks + tiles - 1) / tiles;
  const int64_t min_stages = p->ksplit ? 8 : 4;
  const int64_t max_splits = (p->M + min_stages * bm - 1) / (min_stages * bm);
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t mps = (p->M + splits - 1) / splits;
  mps = (mps + bm - 1) / bm * bm;
  if (mps < bm) mps = bm;
  splits = (p->M + mps - 1) / mps;
  if (splits < 1) splits = 1;
  if (splits * tiles >= INT32_MAX) {
    delete p;
    return FCONV_ERR_UNSUPPORTED;
  }
  p->splits = static_cast<int32_t>(splits);
  p->m_per_split = static_cast<int32_t>(mps);
  p->lp = (p->dw_elems + 3) / 4 * 4;
  p->ws_bytes = splits > 1 ? static_cast<size_t>(splits * p->lp * 4) : 0;
  p->hw_div = make_fast_div(static_cast<uint32_t>(p->Ho * p->Wo));
  p->wo_div = make_fast_div(static_cast<uint32_t>(p->Wo));
  // bf16, 3x3, stride 1, 32-channel input slices and 64-channel output
  // blocks, padded input rows of 33 to 64 pixels: the row-halo kernel, which
  // copies every input and gradient row of its range once.  Ranges of whole
  // output rows, about one workgroup per CU.  Rows of at most 32 pixels (two
  // rows per step, Ho >= 3) only when FCONV_WGRAD_KERNEL=halo pins it: 40.3
  // against 31.0 us for the direct-to-LDS kernel on the 28x28x256 layer, where
  // the 56x56x64 layer takes 22.0 against 25.5-25.9.  FCONV_WGRAD_KERNEL=dma
  // or staged pins the other kernels.
  const bool pin_halo = force && strcmp(force, "halo") == 0;
  p->halo = p->dma && d.dtype == FCONV_BF16 && d.R == 3 && d.S == 3 && d.stride_h == 1 &&
            d.stride_w == 1 && d.C % 32 == 0 && d.K % 64 == 0 && d.W + p->pl + p->pr <= 64 &&
            (p->Wo > 32 || (pin_halo && p->Ho >= 3)) && !(force && strcmp(force, "dma") == 0);
  if (p->halo) {
    p->rps = p->Wo > 32 ? 1 : 2;
    p->tiles_k = d.K / 64;
    p->tiles_kk = d.C / 32;
    const int64_t tl = static_cast<int64_t>(p->tiles_k) * p->tiles_kk;
    const int64_t rows = static_cast<int64_t>(d.N) * p->Ho;
    int64_t sp = kWgTargetBlocks / 2 / tl;
    if (sp > rows) sp = rows;
    if (sp < 1) sp = 1;
    const int64_t rps_split = rows > 0 ? (rows + sp - 1) / sp : 1;  // output rows per range
    sp = rows > 0 ? (rows + rps_split - 1) / rps_split : 1;
    if (sp * tl >= INT32_MAX) {
      delete p;
      return FCONV_ERR_UNSUPPORTED;
    }
    p->splits = static_cast<int32_t>(sp);
    p->m_per_split = static_cast<int32_t>(rps_split);
    p->ws_bytes = sp > 1 ? static_cast<size_t>(sp * p->lp * 4) : 0;
    p->ring = 0;
    p->tk = 64;
    p->ksplit = false;
  }
  p->ho_div = make_fast_div(static_cast<uint32_t>(p->Ho));
  p->kernel_name = wgrad_kernel_name(d.dtype, p->tk, p->vec, p->dma, p->ring, p->ksplit, p->halo);
  // FCONV_LOG=1 (environment): the plan's decisions on stderr.
  const char* lg = getenv("FCONV_LOG");
  if (lg && *lg && strcmp(lg, "0") != 0)
    fprintf(stderr,
            "fconv: wgrad plan N=%d H=%d W=%d C=%d K=%d R=%d S=%d stride=%dx%d %s %s -> Ho=%d "
            "Wo=%d kernel=%s channel_tile=%d ring=%d pixel_ranges=%d (%d pixels each) "
            "workspace=%zu B\n",
            d.N, d.H, d.W, d.C, d.K, d.R, d.S, d.stride_h, d.stride_w, same ? "SAME" : "VALID",
            d.dtype == FCONV_BF16 ? "bf16" : "fp32", p->Ho, p->Wo, p->kernel_name, p->tk, p->ring,
            p->splits, p->m_per_split, p->ws_bytes);
  *out = p;
  return FCONV_OK;
}

fconv_status fconv_wgrad_plan_output_dims(fconv_wgrad_plan p, int32_t* Ho, int32_t* Wo,
                                          int32_t pads_tblr[4]) {
  if (!p) return FCONV_ERR_INVALID_ARG;
  if (Ho) *Ho = p->Ho;
  if (Wo) *Wo = p->Wo;
  if (pads_tblr) {
    pads_tblr[0] = p->pt;
    pads_tblr[1] = p->pb;
    pads_tblr[2] = p->pl;
    pads_tblr[3] = p->pr;
  }
  return FCONV_OK;
}

fconv_status fconv_wgrad_plan_workspace_size(fconv_wgrad_plan p, size_t* bytes) {
  if (!p || !bytes) return FCONV_ERR_INVALID_ARG;
  *bytes = p->ws_bytes;
  return FCONV_OK;
}

fconv_status fconv_wgrad_plan_run(fconv_wgrad_plan p, void* stream, const void* x,
                                  const void* dy, void* dw, void* workspace,
                                  size_t workspace_bytes) {
  using namespace fconv;
  if (!p || !x || !dy || !dw) return FCONV_ERR_INVALID_ARG;
  if (p->ws_bytes > 0 && (!workspace || workspace_bytes < p->ws_bytes)) return FCONV_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dw) ||
      (p->ws_bytes > 0 && !aligned16(workspace)))
    return FCONV_ERR_MISALIGNED;
  const size_t xb = static_cast<size_t>(p->x_elems) * p->esize;
  const size_t db = static_cast<size_t>(p->dy_elems) * p->esize;
  const size_t wb = static_cast<size_t>(p->dw_elems) * (p->out_fp32 ? 4 : 2);
  if (overlaps(dw, wb, x, xb) || overlaps(dw, wb, dy, db) ||
      overlaps(dw, wb, workspace, p->ws_bytes) || overlaps(workspace, p->ws_bytes, x, xb) ||
      overlaps(workspace, p->ws_bytes, dy, db))
    return FCONV_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t L = p->dw_elems;
  const int out_bf16 = p->out_fp32 ? 0 : 1;
  if (p->M == 0) {
    // Empty batch: the gradient is zero.
    return launch_wgrad_reduce(nullptr, dw, 0, p->lp, L, out_bf16, s) == hipSuccess
               ? FCONV_OK
               : FCONV_ERR_DEVICE;
  }
  WgArgs a;
  a.x = x;
  a.dy = dy;
  a.out = p->splits > 1 ? workspace : dw;
  a.N = p->d.N; a.H = p->d.H; a.W = p->d.W; a.C = p->d.C; a.K = p->d.K;
  a.R = p->d.R; a.S = p->d.S; a.sh = p->d.stride_h; a.sw = p->d.stride_w;
  a.pt = p->pt; a.pl = p->pl; a.Ho = p->Ho; a.Wo = p->Wo;
  a.M = static_cast<int32_t>(p->M);
  a.Kg = p->Kg;
  a.tiles_k = p->tiles_k;
  a.tiles_kk = p->tiles_kk;
  a.splits = p->splits;
  a.m_per_split = p->m_per_split;
  a.blocks = p->splits * p->tiles_k * p->tiles_kk;
  a.out_mode = p->splits > 1 ? 0 : (p->out_fp32 ? 1 : 2);
  a.lp = p->lp;
  a.x_bytes = static_cast<uint32_t>(xb);
  a.dy_bytes = static_cast<uint32_t>(db);
  a.hw_mul = p->hw_div.mul; a.hw_add = p->hw_div.add; a.hw_shift = p->hw_div.shift;
  a.wo_mul = p->wo_div.mul; a.wo_add = p->wo_div.add; a.wo_shift = p->wo_div.shift;
  a.wo_ge_e = p->Wo >= p->E;
  a.ho_mul = p->ho_div.mul; a.ho_add = p->ho_div.add; a.ho_shift = p->ho_div.shift;
  hipError_t e = p->d.dtype == FCONV_BF16 ? launch_wgrad_dt<FCONV_BF16>(p, a, s)
                                           : launch_wgrad_dt<FCONV_FP32>(p, a, s);
  if (e != hipSuccess) return FCONV_ERR_DEVICE;
  if (p->splits > 1 && launch_wgrad_reduce(static_cast<const float*>(workspace), dw, p->splits,
                                            p->lp, L, out_bf16, s) != hipSuccess)
    return FCONV_ERR_DEVICE;
  return FCONV_OK;
}

const char* fconv_wgrad_plan_kernel_name(fconv_wgrad_plan p) { return p ? p->kernel_name : nullptr; }

fconv_status fconv_wgrad_plan_destroy(fconv_wgrad_plan p) {
  delete p;
  return FCONV_OK;
}

}  // extern "C"
