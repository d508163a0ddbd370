// Host-side plan object shared by plan.cpp (validation, geometry, variant
// choice; no HIP) and the kernel launchers in conv.hip.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "fconv.h"

namespace fconv {

// Kernel families.  Every plan can fall back to kGeneral; the others are
// shape-specialised tilings chosen by choose_variant() in plan.cpp.
enum Variant : int32_t {
  kGeneral = 0,        // any shape: direct-from-global implicit GEMM, 64x64 tile
  kResidentFilter = 1, // 64-channel filter slice staged in LDS once per workgroup
  kStream = 2,         // int8, short reduction: filter in registers, persistent
  kTiled = 3,          // 128x128 LDS-tiled implicit GEMM, long reductions
  kHalo = 4,           // int8 stride 1 over 64 channels: input rows staged in LDS
  kGemm = 5,           // full-size VALID filter: split-reduction GEMM + sum/epilogue
  kHaloS2 = 6,         // int8 3x3 stride 2 over 64/128 channels: filter in registers, rows in LDS
};

// Division by a runtime constant d for numerators below 2^31:
// n / d = (umulhi(n, mul) + (add ? n : 0)) >> shift.
struct FastDiv {
  uint32_t mul, add, shift;
};
FastDiv make_fast_div(uint32_t d);

// Output size and padding along one axis (SAME or VALID); false for VALID
// with in < f.  Shared by the forward and weight-gradient plans.
bool resolve_axis(int32_t in, int32_t f, int32_t stride, bool same, int32_t* out,
                  int32_t* before, int32_t* after);

// How the implicit-GEMM A operand (im2col row) is gathered, per 16-byte
// chunk of the reduction dimension (r, s, c):
//   kLoadTap:   C is a multiple of one k-step, so a whole k-step sits in one
//               filter tap and the tap loop is uniform across the wave;
//   kLoadChunk: C is a multiple of a 16-byte chunk; one predicated 128-bit
//               load per chunk, tap decoded per lane;
//   kLoadElem:  anything else; element-wise predicated loads.
enum LoadMode : int32_t { kLoadTap = 0, kLoadChunk = 1, kLoadElem = 2 };

}  // namespace fconv

struct fconv_plan_s {
  fconv_desc d;
  int32_t Ho, Wo, pt, pb, pl, pr;
  int32_t esize;       // bytes per x/w/y element
  int32_t chunk_elems; // elements per 16-byte chunk (16 int8, 8 bf16, 4 fp32)
  bool op_scale, op_side, op_bias, op_bn, op_relu;
  bool cudnn7;          // int8 epilogue in the cuDNN 7 order (FCONV_DESC_CUDNN7_ORDER)
  int32_t act;          // float activation: 0 none, 1 ReLU, 2 leaky, 3 clipped, 4 clamp
  int64_t M;      // N * Ho * Wo, rows of the implicit GEMM
  int32_t Kg;     // R * S * C, reduction length
  int32_t KgP;    // Kg rounded up to whole k-steps (4 chunks)
  int32_t Kp;     // K rounded up to a multiple of 64 (packed filter rows)
  int32_t load_mode;
  int32_t variant;
  int32_t pixel_tiles;  // kResidentFilter: 16-pixel MFMA tiles per wave (1, 2, 4);
                        // kTiled: 64-pixel rows of the tile (1, 2, 4; 0 = by grid size)
  int32_t ring_depth;   // kResidentFilter: k-steps of patch loads in flight
  int32_t halo_rows;    // kHalo: output rows per workgroup, 0 = sized to the device
  bool tile_roles;      // kTiled, int8/bf16, 64- or 128-pixel tiles: copy waves beside MFMA waves
  int32_t wrow_bytes;   // packed filter row stride: KgP * esize + 16 (zero pad)
  fconv::FastDiv wo_div, ho_div;
  size_t pack_bytes;    // packed filter: Kp * wrow_bytes
  size_t part_offset;   // kGemm-capable shapes: partial sums after the packed filter (else 0)
  int32_t gemm_splits;  // kGemm: reduction ranges (partial tiles per output)
  int32_t gemm_kps;     // kGemm: 64-byte k-steps per range
  size_t ws_bytes;      // workspace: pack_bytes, then gemm_splits * N * Kp * 4 partial sums (kGemm shapes)
  int64_t x_elems, y_elems, w_elems;
  const char* kernel_name;
};

namespace fconv {
// One kernel configuration of a plan: the family and its tiling knobs.
struct KernelConfig {
  int32_t variant, pixel_tiles, ring_depth, halo_rows;
};
// The configurations that can run the plan's shape, the plan's current one
// first; returns how many were written (at most max).
int list_configs(const fconv_plan_s* p, KernelConfig* out, int max);
// Make `c` the plan's configuration (and kernel name).
void apply_config(fconv_plan_s* p, const KernelConfig& c);
// Process-wide cache of autotuned configurations, keyed by the plan
// descriptor (the operator list past n_ops ignored).
void cache_store(const fconv_desc& d, const KernelConfig& c);

// Argument checks of fconv_plan_run / fconv_plan_pack_filter that need no
// device: pointers, alignment, workspace size, aliasing.  Implemented in
// plan.cpp.
fconv_status check_run_args(const fconv_plan_s* p, const fconv_args* a);
fconv_status check_pack_args(const fconv_plan_s* p, const void* w,
                             const void* workspace, size_t workspace_bytes);
}  // namespace fconv
