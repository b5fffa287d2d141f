// hh_kernels.h -- host-side launchers of the libhh kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hh {

typedef uint16_t bf16_t;

// Map and dtype codes of include/hh.h, for device code that does not include it.
constexpr int HH_MAP_HEDGEHOG_ = 0, HH_MAP_TAYLOR2_ = 1, HH_MAP_HEDGEHOG_SOFTMAX_ = 2, HH_MAP_EXP_ = 3,
              HH_MAP_SOFTMAX_ = 4, HH_MAP_QUADRATIC_ = 5;

// Coefficients of the quadratic kernels a + b s + c s^2 (s = q.k) of one head: the degree-2 Taylor
// map is (1, 1, 1/2); the generalised quadratic map reads (a, b, c) of head h from coef[3 h ..].
// Feature scales: sqrt(a) for the constant, sqrt(b) for x, sqrt(c) for the canonical pair
// features x_i x_j (and so for the packed diagonal x_i^2), sqrt(2 c) for a packed off-diagonal pair.
struct QuadCoef {
    float a, b, c, sa, sb, sc, s2c;
};
__host__ __device__ inline QuadCoef quad_coef(const float *coef, int h) {
    QuadCoef q;
    q.a = coef ? coef[3 * h] : 1.0f;
    q.b = coef ? coef[3 * h + 1] : 1.0f;
    q.c = coef ? coef[3 * h + 2] : 0.5f;
    q.sa = sqrtf(q.a);
    q.sb = sqrtf(q.b);
    q.sc = sqrtf(q.c);
    q.s2c = sqrtf(2.0f * q.c);
    return q;
}
constexpr int HH_F32_ = 0, HH_BF16_ = 1;

// Size of the library-owned scratch array behind hh_linattn_fwd_noalloc (one per device).
constexpr size_t kNoAllocScratchBytes = 64u << 20;
// Device address of that array on the current device (resolved once per device, then cached).
hipError_t noalloc_scratch(void **ptr);

// Chunked Hedgehog kernels (bf16).  Modes: 0 segment state, 1 causal, 2 read-out.
struct WideParams {
    const bf16_t *q, *k, *v, *W, *b;  // b may be null
    bf16_t *y;
    const float *S_in, *z_in;   // starting state (internal row order), or null = zero
    long in_bh_stride;          // slots per (b,h) in S_in
    long in_seg_stride;         // slots per segment in S_in (0: one slot shared by all segments)
    float *S_slots;             // segment slots: S in fp32, in the register-image layout of the
    float *z_slots;             //   kernel that reads them back; z in fp32, feature order
    long slot_bh_stride;        // slots per (b,h)
    float *S_out, *z_out;       // final state (mode 1, last segment), or null
    int N, H, nseg_grid, seg_len;
    int BH;                     // sequences (batch x heads)
    int slot_mode;              // slot added to the starting state of segment s (modes 1, 2):
                                //   0 none, 1 slot s if s > 0 (exclusive prefixes), 2 slot 0 (total),
                                //   3 the sum of slots 0 .. s - 1 (segment aggregates, summed by the
                                //   causal pass itself; no scan)
    int softmax;                // 1: the per-half softmax map (d = 128, no bias), 0: the Hedgehog map
};
// Segment slots of the wide kernels: per (b,h), nseg slots of S (2 d * d floats) and z
// (2 d floats).  Mode 0: aggregates of slots 0 .. nseg-2 become exclusive prefixes in slots
// 1 .. nseg-1; mode 1: the total of all nseg slots goes to slot 0.  Sums run in fp32.
hipError_t launch_slot_scan(int d, float *S_slots, float *z_slots, int BH, int nseg, int mode, hipStream_t st);
hipError_t launch_wide(int d, int mode, const WideParams &p, int grid, hipStream_t st);
// Bidirectional forward with one segment per sequence (d = 64): state and read-out in one
// workgroup per sequence, the total state handed over in LDS (no workspace).
hipError_t launch_bidir_fused(int d, const WideParams &p, int BH, hipStream_t st);
int wide_wgs_per_cu(int d);

// Hedgehog feature map on the matrix cores (bf16): x [BH][N][d] -> phi [BH][N][2d].
hipError_t launch_featuremap_hedgehog_bf16(int d, const bf16_t *x, const bf16_t *W, const bf16_t *b,
                                           bf16_t *phi, int BH, int H, int N, hipStream_t st);

// Degree-2 Taylor chunked kernels (bf16, d = 16).  Modes as above.
struct NarrowParams {
    const bf16_t *q, *k, *v;
    bf16_t *y;
    const float *S_in, *z_in;
    long in_bh_stride, in_seg_stride;
    float *S_ws, *z_ws;
    long ws_bh_stride;
    float *S_out, *z_out;  // canonical feature order
    const float *S0c, *z0c;  // the caller's initial state, canonical order (or null), read only for
                             // the part of S_out the packed basis does not hold
    const float *coef;  // generalised quadratic map: (a, b, c) per head, fp32 [H][3]; null: Taylor
    int N, H, nseg_grid, seg_len;
};
hipError_t launch_narrow(int mode, const NarrowParams &p, int grid, hipStream_t st);
constexpr int kTaylorRowsInternal = 160;  // 153 packed symmetric features padded to 10 blocks of 16

// Scan of segment aggregates into exclusive prefixes (mode 0) or one total (mode 1).
struct PrefixParams {
    float *S_ws, *z_ws;            // [BH][nseg][dpi][d], [BH][nseg][dpi]
    const float *S0, *z0;          // canonical [BH][dpc][d], [BH][dpc] or null
    int BH, nseg, dpi, dpc, d, map, mode;
};
hipError_t launch_prefix(const PrefixParams &p, hipStream_t st);

// S_out = S0 (or 0), z_out = z0 (or 0): the state result of an empty sequence.
hipError_t launch_state_copy(const float *S0, const float *z0, float *S_out, float *z_out, long nS, long nz,
                             hipStream_t st);

// Distillation loss (one workgroup per 128 queries of a (b,h)).  phi_k: the 2d bf16 features of
// k; W, b: the Hedgehog parameters (the kernel maps the queries itself).  Unused for the Taylor map.
struct DistillParams {
    const bf16_t *q, *k, *phi_k, *W, *b;
    float *loss;
    int N, BH, H;
};
hipError_t launch_distill(int map, int d, const DistillParams &p, int BH, hipStream_t st);

// Linear attention over given bf16 features (the maps computed into a workspace first).
// Modes: 0 segment aggregates into slots, 1 causal, 2 read-out against a total (bidirectional).
// Slots: per (b,h) and segment, S [dpp][d] fp32 in the kernel's register image, then z [dpp]
// fp32 (dpp = d' rounded up to a multiple of 32).
struct FeatParams {
    const bf16_t *phiq, *phik, *v;  // [BH][N][d'], [BH][N][d'], [BH][N][d]
    bf16_t *y;
    const float *S0, *z0;           // caller's initial state, canonical [BH][d'][d], [BH][d'] (or null)
    float *S_out, *z_out;           // final state (causal, last segment), canonical (or null)
    float *S_slots, *z_slots;
    long slot_bh_stride;
    int N, seg_len, nseg_grid;
    int slot_mode;                  // 0 none, 1 exclusive prefix in slot s, 2 total in slot 0, 3 sum of slots < s
    int slot_canonical;             // state mode: write S as [dpp][d] row-major instead of the register image
};
hipError_t launch_feat(int d, int dp, int mode, const FeatParams &p, int grid, hipStream_t st);
hipError_t launch_feat_scan(float *S, float *z, int d, int dp, int BH, int nseg, int mode, hipStream_t st);
int feat_wgs_per_cu(int d, int dp);
int feat_padded_dim(int dp);
// Feature maps 2, 3, 4 (softmax over the directions per half, single-sided exp, single-sided
// softmax): bf16 on the matrix cores, fp32 on the vector units.  x [BH][N][d] -> phi [BH][N][d'].
hipError_t launch_featuremap_variant(int map, int dtype, int d, const void *x, const void *W, const void *b, void *phi,
                                     long BH, int H, int N, hipStream_t st);

// Backward of the forward over given features (hh_bwd.hip).  Per sequence bh: phi(q), phi(k)
// [N][d'] bf16; v, y, dy [N][d] bf16; dphi(q), dphi(k) [N][d'] bf16 and den, c [N][2] fp32 written
// by the q-side pass; forward sums S, z and reverse sums R, r per segment in canonical fp32 slots
// ([nseg][dpp][d], [nseg][dpp]).
struct BwdParams {
    const bf16_t *phiq, *phik, *v, *y, *dy, *q, *k, *W, *b;
    bf16_t *dphiq, *dphik;
    float *den_c;
    const float *S_slots, *z_slots;
    float *R_slots, *r_slots;
    bf16_t *dq, *dk, *dv;
    float *dW_parts;               // [BH * wgs_per_seq][d*d + d]
    int N, H, nseg, seg_len;
};
// which = 0: q-side pass, 1: k-side pass (grid = BH * nseg)
hipError_t launch_bwd_pass(int which, int d, int dp, int causal, const BwdParams &p, int grid, hipStream_t st);
hipError_t launch_bwd_map(int map, int d, const BwdParams &p, long BH, hipStream_t st);
hipError_t launch_bwd_reduce(const float *parts, float *dW, float *db, int B, int H, int d, int N, hipStream_t st);
int bwd_wgs_per_seq(int N);

// fp32 path: one workgroup per (b,h) walks the sequence token by token.
struct SeqParams {
    const float *q, *k, *v, *W, *b;
    float *y;
    const float *S0, *z0;
    float *S_out, *z_out;
    int N, H, d, dp, map, causal;
};
hipError_t launch_seq_f32(const SeqParams &p, int BH, hipStream_t st);

// Decode step: one workgroup per (b,h) streams the fp32 state.
struct DecodeParams {
    const void *q, *k, *v, *W, *b;
    void *y;
    float *S, *z;
    int H, d, dp, map, dtype;
};
hipError_t launch_decode(const DecodeParams &p, int BH, hipStream_t st);

// Feature map on the vector units (fp32 Hedgehog, Taylor in either dtype).
hipError_t launch_featuremap_generic(int map, int dtype, int d, int dp, const void *x, const void *W,
                                     const void *b, void *phi, long BH, int H, int N, hipStream_t st);

}  // namespace hh
