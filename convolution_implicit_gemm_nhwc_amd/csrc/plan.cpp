// Plan creation and argument validation (host only, no HIP calls).
//
// The split between a plan (geometry + ordered operators, resolved once) and
// per-run arguments follows MIOpen "Using the fusion API" (sections "Creating
// a fusion plan", "Compiling the fusion plan", "Setting runtime arguments").
// The argument checks mirror the ones TensorFlow conv_ops_fused_int8.cc makes
// before its fused int8 conv (LaunchFusedConv2DOpCpuInt8Helper: no groups,
// NHWC, dilation 1, BiasAdd with or without Relu) but report status codes
// instead of aborting.
#include <limits.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <new>
#include <string>

#include "plan.h"

namespace {

using namespace fconv;

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Accepted operator sequences; see the fconv_op comment in fconv.h.
fconv_status parse_ops(fconv_plan_s* p) {
  const fconv_desc& d = p->d;
  if (d.n_ops < 0 || d.n_ops > FCONV_MAX_OPS) return FCONV_ERR_INVALID_ARG;
  p->op_scale = p->op_side = p->op_bias = p->op_bn = p->op_relu = false;
  p->act = 0;
  int i = 0;
  auto next_is = [&](int32_t op) {
    if (i < d.n_ops && d.ops[i] == op) {
      ++i;
      return true;
    }
    return false;
  };
  if (d.dtype == FCONV_INT8) {
    // TensorFlow conv_ops_fused_int8.cc, BiasActivationOutputKernel: scale,
    // side input, bias, then BiasAdd or BiasAdd+Relu.
    p->op_scale = next_is(FCONV_OP_SCALE);
    p->op_side = next_is(FCONV_OP_SIDE);
    p->op_bias = next_is(FCONV_OP_BIAS);
    p->op_relu = next_is(FCONV_OP_RELU);
    if (!p->op_scale || !p->op_bias) return FCONV_ERR_UNSUPPORTED;
  } else {
    // MIOpen supported fusions: conv -> bias -> batch norm -> activation
    // (Relu, Leaky Relu, Clipped Relu or CLAMP).
    p->op_bias = next_is(FCONV_OP_BIAS);
    p->op_bn = next_is(FCONV_OP_BN);
    p->op_relu = next_is(FCONV_OP_RELU);
    if (p->op_relu) p->act = 1;
    else if (next_is(FCONV_OP_LEAKY_RELU)) p->act = 2;
    else if (next_is(FCONV_OP_CLIPPED_RELU)) p->act = 3;
    else if (next_is(FCONV_OP_CLAMP)) p->act = 4;
  }
  if (i != d.n_ops) return FCONV_ERR_UNSUPPORTED;
  return FCONV_OK;
}

const char* kernel_name(int32_t variant, int32_t dtype) {
  static const char* names[7][3] = {
      {"conv_general_i8", "conv_general_bf16", "conv_general_f32"},
      {"conv_rf_i8", "conv_rf_bf16", "conv_rf_f32"},
      {"conv_stream_i8", "conv_stream_bf16", "conv_stream_f32"},
      {"conv_tile_i8", "conv_tile_bf16", "conv_tile_f32"},
      {"conv_halo_i8", "conv_halo_bf16", "conv_halo_f32"},
      {"conv_gemm_i8", "conv_gemm_bf16", "conv_gemm_f32"},
      {"conv_halo_s2_i8", "conv_halo_s2_bf16", "conv_halo_s2_f32"}};
  return names[variant][dtype];
}

// A filter as large as the image with VALID padding (one output pixel per
// image: the GEMM special case of the fused op), whose image rows are whole
// 64-byte k-steps, in 32-bit buffer extents.
bool gemm_shape(const fconv_plan_s* p) {
  const fconv_desc& d = p->d;
  return d.padding == FCONV_PAD_VALID && d.R == d.H && d.S == d.W &&
         (static_cast<int64_t>(p->Kg) * p->esize) % 64 == 0 &&
         p->x_elems * p->esize < (int64_t{1} << 31) &&
         static_cast<int64_t>(p->pack_bytes) < (int64_t{1} << 31);
}

// The stride-2 row kernel: int8, 3x3, stride 2, 64 or 128 input channels,
// 128-channel output slices, padded input rows of at most 64 pixels (Wo <= 31),
// in 32-bit buffer extents.
bool halo_s2_shape(const fconv_plan_s* p) {
  const fconv_desc& d = p->d;
  return d.dtype == FCONV_INT8 && d.R == 3 && d.S == 3 && d.stride_h == 2 && d.stride_w == 2 &&
         (d.C == 64 || d.C == 128) && d.K % 128 == 0 && p->Wo <= 31 &&
         p->x_elems < (int64_t{1} << 31) && p->y_elems < (int64_t{1} << 31) &&
         static_cast<int64_t>(p->pack_bytes) < (int64_t{1} << 31);
}

// LDS budget of the resident-filter kernel's 64-row filter slice: at most
// this much, so that two workgroups still fit in a CU's 160 KiB.
constexpr int64_t kRfMaxLds = 80 * 1024;

// Kernel choice.  FCONV_FORCE_VARIANT=general|rf|tile|stream|gemm|halo_s2
// (environment) pins a kernel family where the shape allows it, for A/B
// comparisons (a full-size VALID filter takes the GEMM kernel unless another
// family is pinned);
// FCONV_RF_PT=1|2|4 overrides the pixel tiles, FCONV_HALO_ROWS the output rows
// per workgroup of the row-halo kernel, FCONV_TILE_BM=64|128|256 the pixel
// rows of the tiled kernel's tile (otherwise chosen at launch from the grid
// size), FCONV_TILE_ROLES=0 the 8-wave tiled kernel in place of the one with
// copy waves (int8 and bf16; fp32 always runs the 8-wave kernel).
void choose_variant(fconv_plan_s* p) {
  const fconv_desc& d = p->d;
  p->variant = kGeneral;
  p->pixel_tiles = 1;
  p->ring_depth = 0;
  p->halo_rows = 0;
  const char* roles = getenv("FCONV_TILE_ROLES");
  p->tile_roles = d.dtype != FCONV_FP32 && !(roles && atoi(roles) == 0);
  const char* force0 = getenv("FCONV_FORCE_VARIANT");
  if (gemm_shape(p) && (!force0 || strcmp(force0, "gemm") == 0)) {
    p->variant = kGemm;
    p->kernel_name = kernel_name(p->variant, d.dtype);
    return;
  }
  const int64_t rf_lds = 64 * static_cast<int64_t>(p->wrow_bytes);
  const int64_t x_bytes = p->x_elems * p->esize, y_bytes = p->y_elems * p->esize;
  const char* force = getenv("FCONV_FORCE_VARIANT");
  const bool force_general = force && strcmp(force, "general") == 0;
  const bool force_tile = force && strcmp(force, "tile") == 0;
  const bool sizes_ok = x_bytes < (int64_t{1} << 31) && y_bytes < (int64_t{1} << 31) &&
                        static_cast<int64_t>(p->pack_bytes) < (int64_t{1} << 31);
  // Long tap-aligned reductions (more than 9 k-steps of 64 bytes) whose
  // channels fill whole 128-byte stages: the LDS-tiled kernel.
  const bool force_rf = force && strcmp(force, "rf") == 0;
  const int64_t ksteps = p->Kg / (4 * p->chunk_elems);
  const bool tile_ok = (static_cast<int64_t>(d.C) * p->esize) % 128 == 0;
  if (!force_general && !force_rf && p->load_mode == kLoadTap && d.K % 16 == 0 && sizes_ok &&
      tile_ok && (ksteps > 9 || rf_lds > kRfMaxLds || force_tile)) {
    p->variant = kTiled;
    p->pixel_tiles = 0;
    const char* bm = getenv("FCONV_TILE_BM");
    if (bm && atoi(bm) == 64) p->pixel_tiles = 1;
    if (bm && atoi(bm) == 128) p->pixel_tiles = 2;
    if (bm && atoi(bm) == 256) p->pixel_tiles = 4;
  } else if (!force_general && p->load_mode == kLoadTap && d.K % 16 == 0 && rf_lds <= kRfMaxLds &&
      sizes_ok) {
    p->variant = kResidentFilter;
    const int64_t nks = static_cast<int64_t>(p->Kg) / (4 * p->chunk_elems);
    // Pixel tiles per wave vs ring depth: keep every k-step in flight when the
    // reduction is short (3x3 over 64 channels: 9 k-steps), otherwise a
    // 4-deep ring with more pixel reuse of each filter fragment.
    if (nks <= 4) {
      p->pixel_tiles = 2;
      p->ring_depth = 4;
    } else if (nks <= 9) {
      p->pixel_tiles = 2;
      p->ring_depth = 9;
    } else {
      p->pixel_tiles = 4;
      p->ring_depth = 4;
    }
    const char* pt = getenv("FCONV_RF_PT");
    const char* rd = getenv("FCONV_RF_DEPTH");
    if (pt) p->pixel_tiles = atoi(pt);
    if (rd) p->ring_depth = atoi(rd);
    // int8 with a short reduction, in the shapes the streaming kernel is
    // instantiated for (3x3 over 64 channels; 1x1 over 64..512): filter slice
    // in registers.  Its tile split computes block * tiles in 32 bits.
    const bool rf_only = force && strcmp(force, "rf") == 0;
    const int32_t cs = d.C / 64;
    const bool shape_ok = (d.R == 3 && d.S == 3 && cs == 1) ||
                          (d.R == 1 && d.S == 1 && (cs == 1 || cs == 2 || cs == 4 || cs == 8));
    const int64_t tiles = (p->M + 15) / 16;
    if (!rf_only && d.dtype == FCONV_INT8 && shape_ok && tiles * 1024 < (int64_t{1} << 31))
      p->variant = kStream;
    // Stride 1, 3x3 over 64 channels, padded input rows of at most 64 pixels
    // (one 4 KiB LDS slot each): the row-halo kernel, unless the streaming
    // kernel is asked for by name.
    const bool force_stream = force && strcmp(force, "stream") == 0;
    if (p->variant == kStream && !force_stream && d.R == 3 && d.S == 3 && cs == 1 &&
        d.stride_h == 1 && d.stride_w == 1 && d.W + p->pl + p->pr <= 64) {
      p->variant = kHalo;
      const char* hr = getenv("FCONV_HALO_ROWS");
      if (hr && atoi(hr) > 0) p->halo_rows = atoi(hr);
    }
  }
  // 3x3 stride 2 over 64 or 128 channels: the stride-2 row kernel, unless
  // another family is asked for by name.
  if (halo_s2_shape(p) && (!force || strcmp(force, "halo_s2") == 0)) {
    p->variant = kHaloS2;
    p->pixel_tiles = 1;
    p->ring_depth = 0;
    const char* hr = getenv("FCONV_HALO_ROWS");
    if (hr && atoi(hr) > 0) p->halo_rows = atoi(hr);
  }
  p->kernel_name = kernel_name(p->variant, d.dtype);
}

// Shape conditions of each family, as choose_variant applies them.
struct FamilyFit {
  bool rf, tile, stream, halo, gemm, halo_s2;
};

FamilyFit family_fit(const fconv_plan_s* p) {
  const fconv_desc& d = p->d;
  const int64_t rf_lds = 64 * static_cast<int64_t>(p->wrow_bytes);
  const int64_t x_bytes = p->x_elems * p->esize, y_bytes = p->y_elems * p->esize;
  const bool sizes_ok = x_bytes < (int64_t{1} << 31) && y_bytes < (int64_t{1} << 31) &&
                        static_cast<int64_t>(p->pack_bytes) < (int64_t{1} << 31);
  FamilyFit f;
  const bool tap = p->load_mode == kLoadTap && d.K % 16 == 0 && sizes_ok;
  f.tile = tap && (static_cast<int64_t>(d.C) * p->esize) % 128 == 0;
  f.rf = tap && rf_lds <= kRfMaxLds;
  const int32_t cs = d.C / 64;
  const bool shape_ok = (d.R == 3 && d.S == 3 && cs == 1) ||
                        (d.R == 1 && d.S == 1 && (cs == 1 || cs == 2 || cs == 4 || cs == 8));
  const int64_t tiles = (p->M + 15) / 16;
  f.stream = f.rf && d.dtype == FCONV_INT8 && shape_ok && tiles * 1024 < (int64_t{1} << 31);
  f.halo = f.stream && d.R == 3 && d.S == 3 && cs == 1 && d.stride_h == 1 && d.stride_w == 1 &&
           d.W + p->pl + p->pr <= 64;
  f.gemm = gemm_shape(p);
  f.halo_s2 = halo_s2_shape(p);
  return f;
}

fconv_desc cache_key(const fconv_desc& d) {
  fconv_desc k;
  memset(&k, 0, sizeof(k));
  k = d;
  for (int i = d.n_ops < 0 ? 0 : d.n_ops; i < FCONV_MAX_OPS; ++i) k.ops[i] = 0;
  return k;
}

std::mutex& cache_mutex() {
  static std::mutex m;
  return m;
}

std::map<std::string, KernelConfig>& cache_map() {
  static std::map<std::string, KernelConfig> m;
  return m;
}

std::string key_bytes(const fconv_desc& d) {
  const fconv_desc k = cache_key(d);
  return std::string(reinterpret_cast<const char*>(&k), sizeof(k));
}

bool cache_lookup(const fconv_desc& d, KernelConfig* c) {
  std::lock_guard<std::mutex> lock(cache_mutex());
  auto it = cache_map().find(key_bytes(d));
  if (it == cache_map().end()) return false;
  *c = it->second;
  return true;
}

bool aligned(const void* ptr, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// FCONV_LOG=1 (environment): one line on stderr per plan with the decisions
// plan creation made -- geometry, padding, the kernel family and its tiling,
// and the workspace size -- for logs and A/B comparisons.
void log_plan(const fconv_plan_s* p, bool from_cache) {
  const char* lg = getenv("FCONV_LOG");
  if (!lg || !*lg || strcmp(lg, "0") == 0) return;
  const fconv_desc& d = p->d;
  static const char* dt[3] = {"int8", "bf16", "fp32"};
  fprintf(stderr,
          "fconv: plan N=%d H=%d W=%d C=%d K=%d R=%d S=%d stride=%dx%d %s %s -> Ho=%d Wo=%d "
          "pads(t,b,l,r)=%d,%d,%d,%d kernel=%s%s pixel_tiles=%d ring_depth=%d halo_rows=%d "
          "tile_roles=%d gemm_splits=%d workspace=%zu B\n",
          d.N, d.H, d.W, d.C, d.K, d.R, d.S, d.stride_h, d.stride_w,
          d.padding == FCONV_PAD_SAME ? "SAME" : "VALID", dt[d.dtype], p->Ho, p->Wo, p->pt, p->pb,
          p->pl, p->pr, p->kernel_name, from_cache ? " (autotuned)" : "", p->pixel_tiles,
          p->ring_depth, p->halo_rows, p->tile_roles ? 1 : 0, p->gemm_splits, p->ws_bytes);
}

}  // namespace

namespace fconv {

int list_configs(const fconv_plan_s* p, KernelConfig* out, int max) {
  int n = 0;
  auto add = [&](int32_t v, int32_t pt, int32_t rd, int32_t hr) {
    for (int i = 0; i < n; ++i)
      if (out[i].variant == v && out[i].pixel_tiles == pt && out[i].ring_depth == rd &&
          out[i].halo_rows == hr)
        return;
    if (n < max) out[n++] = KernelConfig{v, pt, rd, hr};
  };
  add(p->variant, p->pixel_tiles, p->ring_depth, p->halo_rows);
  const FamilyFit f = family_fit(p);
  if (f.gemm) add(kGemm, 0, 0, 0);
  if (f.halo) add(kHalo, 1, 0, 0);
  if (f.halo_s2) add(kHaloS2, 1, 0, 0);
  if (f.stream) add(kStream, 1, 0, 0);
  if (f.tile) {
    add(kTiled, 0, 0, 0);
    add(kTiled, 1, 0, 0);
    add(kTiled, 2, 0, 0);
    add(kTiled, 4, 0, 0);
  }
  if (f.rf) {
    static const int32_t pt_rd[6][2] = {{1, 4}, {1, 9}, {2, 4}, {2, 9}, {4, 2}, {4, 4}};
    for (const auto& c : pt_rd) add(kResidentFilter, c[0], c[1], 0);
  }
  add(kGeneral, 1, 0, 0);
  return n;
}

void apply_config(fconv_plan_s* p, const KernelConfig& c) {
  p->variant = c.variant;
  p->pixel_tiles = c.pixel_tiles;
  p->ring_depth = c.ring_depth;
  p->halo_rows = c.halo_rows;
  p->kernel_name = kernel_name(c.variant, p->d.dtype);
}

void cache_store(const fconv_desc& d, const KernelConfig& c) {
  std::lock_guard<std::mutex> lock(cache_mutex());
  cache_map()[key_bytes(d)] = c;
}

// s = ceil(log2 d), m = floor(2^(32+s) / d) + 1 (< 2^33).  For n < 2^31,
// n*m / 2^(32+s) exceeds n/d by less than 2^-(s+1) <= 1/(2d), which never
// reaches the next integer, so the floor is exact.
FastDiv make_fast_div(uint32_t d) {
  uint32_t s = 0;
  while ((uint64_t{1} << s) < d) ++s;
  const uint64_t m = ((uint64_t{1} << (32 + s)) / d) + 1;
  return FastDiv{static_cast<uint32_t>(m), static_cast<uint32_t>(m >> 32), s};
}

// Output size and padding.  SAME: TensorFlow conv_ops_fused_int8.cc,
// LaunchFusedConv2DOpGpuInt8Helper -- the total padding is
// max(0, (out-1)*stride + filter - in), half of it (rounded down) before and
// the rest after; the output size is ceil(in / stride).  VALID: no padding.
bool resolve_axis(int32_t in, int32_t f, int32_t stride, bool same, int32_t* out,
                  int32_t* before, int32_t* after) {
  if (same) {
    int64_t o = (static_cast<int64_t>(in) + stride - 1) / stride;
    int64_t total = (o - 1) * stride + f - in;
    if (total < 0) total = 0;
    *out = static_cast<int32_t>(o);
    *before = static_cast<int32_t>(total / 2);
    *after = static_cast<int32_t>(total - total / 2);
    return true;
  }
  if (in < f) return false;
  *out = (in - f) / stride + 1;
  *before = *after = 0;
  return true;
}

fconv_status check_pack_args(const fconv_plan_s* p, const void* w,
                             const void* workspace, size_t workspace_bytes) {
  if (!p || !w) return FCONV_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < p->ws_bytes) return FCONV_ERR_WORKSPACE;
  if (!aligned(w, 16) || !aligned(workspace, 16)) return FCONV_ERR_MISALIGNED;
  if (overlap(w, static_cast<size_t>(p->w_elems) * p->esize, workspace, p->ws_bytes))
    return FCONV_ERR_INVALID_ARG;
  return FCONV_OK;
}

fconv_status check_run_args(const fconv_plan_s* p, const fconv_args* a) {
  if (!p || !a) return FCONV_ERR_INVALID_ARG;
  if (a->flags & ~FCONV_RUN_FILTER_PREPACKED) return FCONV_ERR_UNSUPPORTED;
  const bool prepacked = (a->flags & FCONV_RUN_FILTER_PREPACKED) != 0;
  if (!a->x || !a->y) return FCONV_ERR_INVALID_ARG;
  if (!prepacked && !a->w) return FCONV_ERR_INVALID_ARG;
  if (p->op_bias && !a->bias) return FCONV_ERR_INVALID_ARG;
  if (p->op_side && !a->side) return FCONV_ERR_INVALID_ARG;
  if (p->op_bn && (!a->bn_gamma || !a->bn_beta || !a->bn_mean || !a->bn_var))
    return FCONV_ERR_INVALID_ARG;
  if (a->conv_input_scales && !p->op_scale) return FCONV_ERR_UNSUPPORTED;
  if (p->act >= 2) {
    const float al = a->activ_alpha, be = a->activ_beta;
    if (!(al - al == 0.0f)) return FCONV_ERR_INVALID_ARG;  // NaN or infinite
    if (p->act == 4 && !(be - be == 0.0f && al <= be)) return FCONV_ERR_INVALID_ARG;
  }
  if (!a->workspace || a->workspace_bytes < p->ws_bytes) return FCONV_ERR_WORKSPACE;
  if (!aligned(a->x, 16) || !aligned(a->y, 16) || !aligned(a->workspace, 16) ||
      (!prepacked && !aligned(a->w, 16)) || (p->op_side && !aligned(a->side, 16)))
    return FCONV_ERR_MISALIGNED;
  const float* vecs[6] = {p->op_bias ? a->bias : nullptr,
                          p->op_bn ? a->bn_gamma : nullptr,
                          p->op_bn ? a->bn_beta : nullptr,
                          p->op_bn ? a->bn_mean : nullptr,
                          p->op_bn ? a->bn_var : nullptr,
                          a->conv_input_scales};
  for (const float* v : vecs)
    if (v && !aligned(v, 4)) return FCONV_ERR_MISALIGNED;
  // No in-place operation: y may not overlap anything the run reads, nor the
  // workspace it writes.
  const size_t yb = static_cast<size_t>(p->y_elems) * p->esize;
  const size_t xb = static_cast<size_t>(p->x_elems) * p->esize;
  const size_t wb = static_cast<size_t>(p->w_elems) * p->esize;
  if (overlap(a->y, yb, a->x, xb) || overlap(a->y, yb, a->workspace, p->ws_bytes) ||
      (!prepacked && overlap(a->y, yb, a->w, wb)) ||
      (p->op_side && overlap(a->y, yb, a->side, static_cast<size_t>(p->y_elems))))
    return FCONV_ERR_INVALID_ARG;
  if (!prepacked && overlap(a->w, wb, a->workspace, p->ws_bytes))
    return FCONV_ERR_INVALID_ARG;
  return FCONV_OK;
}

}  // namespace fconv

extern "C" {

fconv_status fconv_plan_create(const fconv_desc* desc, fconv_plan* out) {
  if (!desc || !out) return FCONV_ERR_INVALID_ARG;
  *out = nullptr;
  const fconv_desc& d = *desc;
  if (d.dtype != FCONV_INT8 && d.dtype != FCONV_BF16 && d.dtype != FCONV_FP32)
    return FCONV_ERR_UNSUPPORTED;
  if (d.padding != FCONV_PAD_SAME && d.padding != FCONV_PAD_VALID)
    return FCONV_ERR_UNSUPPORTED;
  if (d.flags & ~FCONV_DESC_CUDNN7_ORDER) return FCONV_ERR_UNSUPPORTED;
  if ((d.flags & FCONV_DESC_CUDNN7_ORDER) && d.dtype != FCONV_INT8) return FCONV_ERR_UNSUPPORTED;
  if (d.N < 0 || d.H < 1 || d.W < 1 || d.C < 1 || d.K < 1 || d.R < 1 || d.S < 1 ||
      d.stride_h < 1 || d.stride_w < 1)
    return FCONV_ERR_INVALID_ARG;

  fconv_plan_s* p = new (std::nothrow) fconv_plan_s();
  if (!p) return FCONV_ERR_INVALID_ARG;
  p->d = d;
  p->cudnn7 = (d.flags & FCONV_DESC_CUDNN7_ORDER) != 0;
  const bool same = d.padding == FCONV_PAD_SAME;
  if (!resolve_axis(d.H, d.R, d.stride_h, same, &p->Ho, &p->pt, &p->pb) ||
      !resolve_axis(d.W, d.S, d.stride_w, same, &p->Wo, &p->pl, &p->pr)) {
    delete p;
    return FCONV_ERR_INVALID_ARG;
  }
  fconv_status st = parse_ops(p);
  if (st != FCONV_OK) {
    delete p;
    return st;
  }
  p->esize = d.dtype == FCONV_INT8 ? 1 : d.dtype == FCONV_BF16 ? 2 : 4;
  p->chunk_elems = 16 / p->esize;
  p->x_elems = static_cast<int64_t>(d.N) * d.H * d.W * d.C;
  p->M = static_cast<int64_t>(d.N) * p->Ho * p->Wo;
  p->y_elems = p->M * d.K;
  p->w_elems = static_cast<int64_t>(d.R) * d.S * d.C * d.K;
  const int64_t kg = static_cast<int64_t>(d.R) * d.S * d.C;
  const int64_t kstep = 4 * p->chunk_elems;
  const int64_t kgp = round_up(kg, kstep);
  const int64_t kp = round_up(d.K, 64);
  // Kernels index with 32-bit element offsets.
  if (p->x_elems >= INT32_MAX || p->y_elems >= INT32_MAX || kp * kgp >= INT32_MAX ||
      p->M >= INT32_MAX) {
    delete p;
    return FCONV_ERR_UNSUPPORTED;
  }
  p->Kg = static_cast<int32_t>(kg);
  p->KgP = static_cast<int32_t>(kgp);
  p->Kp = static_cast<int32_t>(kp);
  p->wrow_bytes = static_cast<int32_t>(kgp * p->esize + 16);
  p->pack_bytes = static_cast<size_t>(kp * p->wrow_bytes);
  p->ws_bytes = p->pack_bytes;
  p->part_offset = 0;
  p->gemm_splits = p->gemm_kps = 0;
  if (gemm_shape(p)) {
    // Split the reduction so that 32-channel tiles x 32-image tiles x ranges
    // come to at least one workgroup per CU (256 on the MI355X), with at
    // least 16 k-steps (one per wave) in a range.
    const int64_t nks = kg * p->esize / 64;
    const int64_t tiles = (kp / 32) * ((d.N + 31) / 32);
    int64_t splits = 1;
    while (splits * tiles < 256 && nks / (2 * splits) >= 16) splits *= 2;
    p->gemm_splits = static_cast<int32_t>(splits);
    p->gemm_kps = static_cast<int32_t>((nks + splits - 1) / splits);
    p->part_offset = static_cast<size_t>(round_up(static_cast<int64_t>(p->pack_bytes), 256));
    p->ws_bytes = p->part_offset + static_cast<size_t>(splits) * d.N * kp * 4;
  }
  if (d.C % kstep == 0)
    p->load_mode = kLoadTap;
  else if (d.C % p->chunk_elems == 0)
    p->load_mode = kLoadChunk;
  else
    p->load_mode = kLoadElem;
  p->wo_div = make_fast_div(static_cast<uint32_t>(p->Wo));
  p->ho_div = make_fast_div(static_cast<uint32_t>(p->Ho));
  choose_variant(p);
  // A configuration autotuned earlier in this process for the same
  // descriptor wins, unless a family is pinned through the environment.
  KernelConfig cached;
  const bool from_cache = !getenv("FCONV_FORCE_VARIANT") && cache_lookup(p->d, &cached);
  if (from_cache) apply_config(p, cached);
  log_plan(p, from_cache);
  *out = p;
  return FCONV_OK;
}

fconv_status fconv_plan_output_dims(fconv_plan p, int32_t* Ho, int32_t* Wo,
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

fconv_status fconv_plan_workspace_size(fconv_plan p, size_t* bytes) {
  if (!p || !bytes) return FCONV_ERR_INVALID_ARG;
  *bytes = p->ws_bytes;
  return FCONV_OK;
}

fconv_status fconv_plan_destroy(fconv_plan p) {
  delete p;
  return FCONV_OK;
}

const char* fconv_plan_kernel_name(fconv_plan p) { return p ? p->kernel_name : nullptr; }

void fconv_autotune_cache_clear(void) {
  std::lock_guard<std::mutex> lock(cache_mutex());
  cache_map().clear();
}

const char* fconv_status_string(fconv_status s) {
  // A C caller may pass any int; reading it as the C++ enum type would be
  // undefined for values outside the enumerators' range, so copy the bits.
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case FCONV_OK: return "ok";
    case FCONV_ERR_INVALID_ARG: return "invalid argument";
    case FCONV_ERR_UNSUPPORTED: return "unsupported";
    case FCONV_ERR_WORKSPACE: return "workspace missing or too small";
    case FCONV_ERR_MISALIGNED: return "misaligned pointer";
    case FCONV_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

}  // extern "C"
