// hh_api.cpp -- the C ABI of libhh (include/hh.h): argument checks on the host, planning of
// the segment split and workspace, and kernel dispatch on the caller's stream.
//
// Every check runs before the first HIP call, so invalid arguments return an error with
// nothing enqueued (and without touching the GPU at all).
#include "hh.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "hh_kernels.h"

namespace {

thread_local std::string g_last_error;

hh_status_t fail(hh_status_t st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
hh_status_t fail(hh_status_t st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

hh_status_t ok() {
    g_last_error.clear();
    return HH_OK;
}

// The runtime's last-error slot may still hold a failure from an unrelated earlier call in
// the process (another library probing devices); drop it so that the check after our own
// launches reports only our launches.
void clear_stale_hip_error() { (void)hipGetLastError(); }

hh_status_t hip_fail(hipError_t e, const char *what) {
    return fail(HH_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

int feature_dim(int map, int d) {
    if (d < 1 || d > 1024) return -1;
    if (map == HH_MAP_HEDGEHOG || map == HH_MAP_HEDGEHOG_SOFTMAX) return 2 * d;
    if (map == HH_MAP_TAYLOR2 || map == HH_MAP_QUADRATIC) return 1 + d + d * d;
    if (map == HH_MAP_EXP || map == HH_MAP_SOFTMAX) return d;
    return -1;
}

// Maps with a W (every map but the Taylor map; the generalised quadratic map's W is its fp32
// coefficients [H][3]), and maps with a bias (the softmax maps have none).
bool map_has_W(int map) { return map != HH_MAP_TAYLOR2; }
// The quadratic kernels a + b s + c s^2 (Taylor and the generalised quadratic map): head dim 16,
// the packed-state kernels.
bool quadratic_family(int map) { return map == HH_MAP_TAYLOR2 || map == HH_MAP_QUADRATIC; }
bool map_has_b(int map) { return map == HH_MAP_HEDGEHOG || map == HH_MAP_EXP; }
// Maps whose features the attention kernels read from a workspace (computed by the feature-map
// kernel first) rather than computing them from q and k themselves.
bool map_via_features(int map) { return map == HH_MAP_HEDGEHOG_SOFTMAX || map == HH_MAP_EXP || map == HH_MAP_SOFTMAX; }
// The per-half softmax map in the causal bf16 forward at d = 64 and 128 runs on the Hedgehog
// kernels, which form and normalise the features themselves (no feature tensors in memory).
bool softmax_fused(int map, int dtype, int causal, int d) {
    return map == HH_MAP_HEDGEHOG_SOFTMAX && dtype == HH_BF16 && causal == 1 && (d == 128 || d == 64);
}
// Forwards whose features the kernels read from the workspace.
bool fwd_via_features(int map, int dtype, int causal, int d) {
    return map_via_features(map) && !softmax_fused(map, dtype, causal, d);
}

size_t elem_bytes(int dtype) { return dtype == HH_BF16 ? 2 : 4; }

// Checks shared by the forward and the feature map.
hh_status_t check_common(int map, int dtype, long B, long H, long N, int d) {
    if (map < HH_MAP_HEDGEHOG || map > HH_MAP_QUADRATIC) return fail(HH_EINVAL, "unknown map %d", map);
    if (dtype != HH_F32 && dtype != HH_BF16) return fail(HH_EINVAL, "unknown dtype %d", dtype);
    if (B < 1 || H < 1) return fail(HH_EINVAL, "B and H must be >= 1 (got B=%ld H=%ld)", B, H);
    if (B * H >= (1L << 24)) return fail(HH_EINVAL, "B*H = %ld exceeds 2^24", B * H);
    if (N < 0) return fail(HH_EINVAL, "N must be >= 0 (got %ld)", N);
    if (!quadratic_family(map)) {
        if (d != 16 && d != 32 && d != 64 && d != 128)
            return fail(HH_EUNSUPPORTED, "head dim %d not supported for map %d (16, 32, 64, 128)", d, map);
    } else if (d != 16) {
        return fail(HH_EUNSUPPORTED, "quadratic-kernel map %d: head dim %d not supported (16)", map, d);
    }
    if (N * (long)d >= (1L << 31)) return fail(HH_EINVAL, "N*d = %ld exceeds 2^31", N * (long)d);
    return HH_OK;
}

hh_status_t check_ptr(const void *p, const char *name, bool required) {
    if (!p) return required ? fail(HH_EINVAL, "%s is NULL", name) : HH_OK;
    if (!aligned16(p)) return fail(HH_EINVAL, "%s is not 16-byte aligned", name);
    return HH_OK;
}

// W and b of a map: W required (when there is work) for every map with a W; b optional where the
// map has a bias, and must be NULL for the softmax maps (which omit it) and the Taylor map.
hh_status_t check_params(int map, const void *W, const void *b, bool need) {
    hh_status_t st;
    if (map_has_W(map)) {
        if ((st = check_ptr(W, "W", need)) != HH_OK) return st;
    }
    if (map_has_b(map)) return check_ptr(b, "b", false);
    if (map_has_W(map) && b) return fail(HH_EINVAL, "map %d has no bias: b must be NULL", map);
    return HH_OK;
}

// Workspace of the features-given path: phi(q), phi(k) (bf16), then the segment slots.
struct FeatPlan {
    int dp = 0, dpp = 0, nseg = 1, seg_len = 0;
    size_t off_phik = 0, off_slots = 0, off_z = 0, bytes = 0;
};

FeatPlan make_feat_plan(int map, int causal, long BH, long N, int d) {
    FeatPlan f;
    f.dp = feature_dim(map, d);
    f.dpp = hh::feat_padded_dim(f.dp);
    const long C = 64;
    const long nch = (N + C - 1) / C;
    long nseg = 256L * hh::feat_wgs_per_cu(d, f.dp) / BH;
    if (nseg < 1) nseg = 1;
    if (nseg > nch) nseg = nch;
    const long seg_chunks = nch > 0 ? (nch + nseg - 1) / nseg : 1;
    nseg = nch > 0 ? (nch + seg_chunks - 1) / seg_chunks : 1;
    f.nseg = (int)nseg;
    f.seg_len = (int)(seg_chunks * C);
    const size_t phi = ((size_t)BH * N * f.dp * sizeof(uint16_t) + 255) / 256 * 256;
    f.off_phik = phi;
    f.off_slots = 2 * phi;
    const bool slots = !causal || f.nseg > 1;
    f.off_z = f.off_slots + (slots ? (size_t)BH * f.nseg * f.dpp * d * sizeof(float) : 0);
    f.bytes = f.off_z + (slots ? (size_t)BH * f.nseg * f.dpp * sizeof(float) : 0);
    return f;
}

// ---- planning of the chunked bf16 path -------------------------------------------------
struct Plan {
    bool chunked = false;  // bf16 chunked kernels (else the fp32 token path)
    bool narrow = false;   // Taylor kernels
    int dpi = 0;           // feature rows of the internal state
    int nseg = 1, seg_len = 0;
    bool need_ws = false;  // segment slots in the workspace
    size_t ws_bytes = 0;
};

// Bytes of the fp32 S part of the wide kernels' segment slots (a multiple of 16).
size_t wide_slot_S_bytes(long BH, long nseg, int d) { return (size_t)BH * nseg * 2 * d * d * sizeof(float); }

Plan make_plan(int map, int dtype, int causal, long BH, long N, int d, bool has_S0) {
    Plan pl;
    if (dtype != HH_BF16 || N == 0) return pl;
    pl.chunked = true;
    pl.narrow = quadratic_family(map);
    pl.dpi = pl.narrow ? hh::kTaylorRowsInternal : 2 * d;
    // causal d = 64 runs two sequences per workgroup in 32-token chunks: segments in 32-token
    // steps, about two sequence segments per CU
    const bool pairs = causal && !pl.narrow && d == 64;
    const long C = pairs ? 32 : 64;
    const long nch = (N + C - 1) / C;
    const long target = pl.narrow ? 1024 : pairs ? 512 : 256L * hh::wide_wgs_per_cu(d);
    long nseg = target / BH;
    if (nseg < 1) nseg = 1;
    if (nseg > nch) nseg = nch;
    const long seg_chunks = (nch + nseg - 1) / nseg;
    nseg = (nch + seg_chunks - 1) / seg_chunks;
    pl.nseg = (int)nseg;
    pl.seg_len = (int)(seg_chunks * C);
    if (!causal) pl.need_ws = true;
    else if (pl.nseg > 1) pl.need_ws = true;
    else if (pl.narrow && has_S0) pl.need_ws = true;  // S0 must be reordered into the internal rows
    if (pl.need_ws)
        pl.ws_bytes = pl.narrow ? (size_t)BH * pl.nseg * ((size_t)pl.dpi * d + pl.dpi) * sizeof(float)
                                : wide_slot_S_bytes(BH, pl.nseg, d) + (size_t)BH * pl.nseg * pl.dpi * sizeof(float);
    return pl;
}

// Workspace of the backward: phi(q), phi(k) bf16, dphi(q), dphi(k) fp32, den and c per token,
// forward and reverse segment sums (canonical fp32 slots), and the parts of dW, db.
struct BwdPlan {
    int dp = 0, dpp = 0, nseg = 1, seg_len = 0, wgs = 0;
    size_t off_phik, off_dphiq, off_dphik, off_denc, off_S, off_z, off_R, off_r, off_parts, bytes = 0;
};

BwdPlan make_bwd_plan(int map, long BH, long N, int d) {
    BwdPlan f;
    f.dp = feature_dim(map, d);
    f.dpp = hh::feat_padded_dim(f.dp);
    const long C = 64, nch = (N + C - 1) / C;
    long nseg = 256L / BH;  // one workgroup of d / 16 waves per segment
    if (nseg < 1) nseg = 1;
    if (nseg > nch) nseg = nch;
    const long seg_chunks = (nch + nseg - 1) / nseg;
    nseg = (nch + seg_chunks - 1) / seg_chunks;
    f.nseg = (int)nseg;
    f.seg_len = (int)(seg_chunks * C);
    f.wgs = hh::bwd_wgs_per_seq((int)N);
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t phi = up((size_t)BH * N * f.dp * 2), dphi = phi;
    const size_t slotS = up((size_t)BH * nseg * f.dpp * d * 4), slotz = up((size_t)BH * nseg * f.dpp * 4);
    f.off_phik = phi;
    f.off_dphiq = 2 * phi;
    f.off_dphik = f.off_dphiq + dphi;
    f.off_denc = f.off_dphik + dphi;
    f.off_S = f.off_denc + up((size_t)BH * N * 8);
    f.off_z = f.off_S + slotS;
    f.off_R = f.off_z + slotz;
    f.off_r = f.off_R + slotS;
    f.off_parts = f.off_r + slotz;
    f.bytes = f.off_parts + up((size_t)BH * f.wgs * ((size_t)d * d + d) * 4);
    return f;
}

}  // namespace

extern "C" {

int hh_abi_version(void) { return 1; }

int hh_feature_dim(int map, int d) { return feature_dim(map, d); }

const char *hh_status_str(int s) {
    switch (s) {
    case HH_OK: return "HH_OK: success";
    case HH_EINVAL: return "HH_EINVAL: invalid argument";
    case HH_EUNSUPPORTED: return "HH_EUNSUPPORTED: unsupported configuration";
    case HH_EWORKSPACE: return "HH_EWORKSPACE: workspace missing or too small";
    case HH_EHIP: return "HH_EHIP: HIP runtime error";
    default: return "unknown hh status";
    }
}

const char *hh_last_error(void) { return g_last_error.c_str(); }

hh_status_t hh_featuremap(int map, int dtype, int B, int H, int N, int d, const void *x, const void *W,
                          const void *b, void *phi, void *stream) {
    hh_status_t st = check_common(map, dtype, B, H, N, d);
    if (st != HH_OK) return st;
    const bool hog = map == HH_MAP_HEDGEHOG;
    const int dp = feature_dim(map, d);
    const size_t eb = elem_bytes(dtype);
    if ((st = check_ptr(x, "x", N > 0)) != HH_OK) return st;
    if ((st = check_ptr(phi, "phi", N > 0)) != HH_OK) return st;
    if ((st = check_params(map, W, b, true)) != HH_OK) return st;
    const size_t nx = (size_t)B * H * N * d * eb, nphi = (size_t)B * H * N * dp * eb;
    if (overlap(x, nx, phi, nphi)) return fail(HH_EINVAL, "phi overlaps x");
    if (N == 0) return ok();
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    clear_stale_hip_error();
    hipError_t e;
    if (map_via_features(map))
        e = hh::launch_featuremap_variant(map, dtype, d, x, W, b, phi, (long)B * H, H, N, s);
    else if (hog && dtype == HH_BF16)
        e = hh::launch_featuremap_hedgehog_bf16(d, (const hh::bf16_t *)x, (const hh::bf16_t *)W,
                                                (const hh::bf16_t *)b, (hh::bf16_t *)phi, B * H, H, N, s);
    else
        e = hh::launch_featuremap_generic(map, dtype, d, dp, x, (hog || map == HH_MAP_QUADRATIC) ? W : nullptr,
                                          hog ? b : nullptr, phi,
                                          (long)B * H, H, N, s);
    if (e != hipSuccess) return hip_fail(e, "feature map launch");
    return ok();
}

size_t hh_linattn_fwd_workspace(int map, int dtype, int causal, int B, int H, int N, int d) {
    if (check_common(map, dtype, B, H, N, d) != HH_OK || (causal != 0 && causal != 1)) return 0;
    if (fwd_via_features(map, dtype, causal, d))
        return (dtype == HH_BF16 && N > 0) ? make_feat_plan(map, causal, (long)B * H, N, d).bytes : 0;
    // the larger of the plans with and without an initial state
    const Plan a = make_plan(map, dtype, causal, (long)B * H, N, d, false);
    const Plan b = make_plan(map, dtype, causal, (long)B * H, N, d, true);
    return a.ws_bytes > b.ws_bytes ? a.ws_bytes : b.ws_bytes;
}

hh_status_t hh_linattn_fwd(int map, int dtype, int causal, int B, int H, int N, int d, const void *q,
                           const void *k, const void *v, const void *W, const void *b, const float *S0,
                           const float *z0, void *y, float *S_out, float *z_out, void *workspace,
                           size_t workspace_bytes, void *stream) {
    hh_status_t st = check_common(map, dtype, B, H, N, d);
    if (st != HH_OK) return st;
    if (causal != 0 && causal != 1) return fail(HH_EINVAL, "causal must be 0 or 1 (got %d)", causal);
    const int dp = feature_dim(map, d);
    const long BH = (long)B * H;
    const size_t eb = elem_bytes(dtype);
    const bool need_io = N > 0;
    if ((st = check_ptr(q, "q", need_io)) != HH_OK) return st;
    if ((st = check_ptr(k, "k", need_io)) != HH_OK) return st;
    if ((st = check_ptr(v, "v", need_io)) != HH_OK) return st;
    if ((st = check_ptr(y, "y", need_io)) != HH_OK) return st;
    if ((st = check_params(map, W, b, need_io)) != HH_OK) return st;
    if ((S0 == nullptr) != (z0 == nullptr)) return fail(HH_EINVAL, "S0 and z0 must be both set or both NULL");
    if ((S_out == nullptr) != (z_out == nullptr))
        return fail(HH_EINVAL, "S_out and z_out must be both set or both NULL");
    if (!causal && (S0 || S_out)) return fail(HH_EINVAL, "initial/final state is only defined for causal attention");
    if ((st = check_ptr(S0, "S0", false)) != HH_OK) return st;
    if ((st = check_ptr(z0, "z0", false)) != HH_OK) return st;
    if ((st = check_ptr(S_out, "S_out", false)) != HH_OK) return st;
    if ((st = check_ptr(z_out, "z_out", false)) != HH_OK) return st;
    const size_t nio = (size_t)BH * N * d * eb;
    if (overlap(y, nio, q, nio) || overlap(y, nio, k, nio) || overlap(y, nio, v, nio))
        return fail(HH_EINVAL, "y overlaps q, k or v");
    const size_t nS = (size_t)BH * dp * d * sizeof(float), nz = (size_t)BH * dp * sizeof(float);
    if (overlap(y, nio, S_out, nS) || overlap(y, nio, z_out, nz)) return fail(HH_EINVAL, "y overlaps S_out or z_out");

    if (fwd_via_features(map, dtype, causal, d) && dtype == HH_BF16 && N > 0) {
        const FeatPlan fp = make_feat_plan(map, causal, BH, N, d);
        if (!workspace) return fail(HH_EWORKSPACE, "workspace of %zu bytes required, got NULL", fp.bytes);
        if (workspace_bytes < fp.bytes)
            return fail(HH_EWORKSPACE, "workspace of %zu bytes required, got %zu", fp.bytes, workspace_bytes);
        if (!aligned16(workspace)) return fail(HH_EINVAL, "workspace is not 16-byte aligned");
        if (overlap(workspace, fp.bytes, y, nio) || overlap(workspace, fp.bytes, q, nio) ||
            overlap(workspace, fp.bytes, k, nio) || overlap(workspace, fp.bytes, v, nio))
            return fail(HH_EINVAL, "workspace overlaps an input or output");
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        clear_stale_hip_error();
        char *ws = reinterpret_cast<char *>(workspace);
        hh::bf16_t *phiq = reinterpret_cast<hh::bf16_t *>(ws), *phik = reinterpret_cast<hh::bf16_t *>(ws + fp.off_phik);
        hipError_t e = hh::launch_featuremap_variant(map, dtype, d, q, W, b, phiq, BH, H, N, s);
        if (e == hipSuccess) e = hh::launch_featuremap_variant(map, dtype, d, k, W, b, phik, BH, H, N, s);
        if (e != hipSuccess) return hip_fail(e, "feature map launch");
        hh::FeatParams f;
        memset(&f, 0, sizeof f);
        f.phiq = phiq; f.phik = phik; f.v = (const hh::bf16_t *)v; f.y = (hh::bf16_t *)y;
        f.S_slots = reinterpret_cast<float *>(ws + fp.off_slots);
        f.z_slots = reinterpret_cast<float *>(ws + fp.off_z);
        f.slot_bh_stride = fp.nseg;
        f.N = N; f.seg_len = fp.seg_len;
        const bool direct = fp.nseg <= 8;
        if (causal) {
            if (fp.nseg > 1) {
                f.nseg_grid = fp.nseg - 1;
                e = hh::launch_feat(d, fp.dp, 0, f, (int)(BH * (fp.nseg - 1)), s);
                if (e == hipSuccess && !direct) e = hh::launch_feat_scan(f.S_slots, f.z_slots, d, fp.dp, (int)BH, fp.nseg, 0, s);
                if (e != hipSuccess) return hip_fail(e, "segment-state launch");
            }
            f.slot_mode = fp.nseg > 1 ? (direct ? 3 : 1) : 0;
            f.S0 = S0; f.z0 = z0; f.S_out = S_out; f.z_out = z_out;
            f.nseg_grid = fp.nseg;
            e = hh::launch_feat(d, fp.dp, 1, f, (int)(BH * fp.nseg), s);
        } else {
            f.nseg_grid = fp.nseg;
            e = hh::launch_feat(d, fp.dp, 0, f, (int)(BH * fp.nseg), s);
            if (e == hipSuccess && fp.nseg > 1) e = hh::launch_feat_scan(f.S_slots, f.z_slots, d, fp.dp, (int)BH, fp.nseg, 1, s);
            if (e != hipSuccess) return hip_fail(e, "segment-state launch");
            f.slot_mode = 2;
            e = hh::launch_feat(d, fp.dp, 2, f, (int)(BH * fp.nseg), s);
        }
        if (e != hipSuccess) return hip_fail(e, "chunked forward launch");
        return ok();
    }

    const Plan pl = make_plan(map, dtype, causal, BH, N, d, S0 != nullptr);
    if (pl.need_ws) {
        if (!workspace) return fail(HH_EWORKSPACE, "workspace of %zu bytes required, got NULL", pl.ws_bytes);
        if (workspace_bytes < pl.ws_bytes)
            return fail(HH_EWORKSPACE, "workspace of %zu bytes required, got %zu", pl.ws_bytes, workspace_bytes);
        if (!aligned16(workspace)) return fail(HH_EINVAL, "workspace is not 16-byte aligned");
        if (overlap(workspace, pl.ws_bytes, y, nio) || overlap(workspace, pl.ws_bytes, q, nio) ||
            overlap(workspace, pl.ws_bytes, k, nio) || overlap(workspace, pl.ws_bytes, v, nio))
            return fail(HH_EINVAL, "workspace overlaps an input or output");
    }

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    clear_stale_hip_error();
    hipError_t e = hipSuccess;
    if (N == 0) {
        if (S_out) e = hh::launch_state_copy(S0, z0, S_out, z_out, (long)BH * dp * d, (long)BH * dp, s);
        if (e != hipSuccess) return hip_fail(e, "state copy launch");
        return ok();
    }

    if (!pl.chunked) {  // fp32 token-by-token path
        hh::SeqParams sp;
        sp.q = (const float *)q; sp.k = (const float *)k; sp.v = (const float *)v;
        sp.W = map_has_W(map) ? (const float *)W : nullptr;
        sp.b = map_has_b(map) ? (const float *)b : nullptr;
        sp.y = (float *)y;
        sp.S0 = S0; sp.z0 = z0; sp.S_out = S_out; sp.z_out = z_out;
        sp.N = N; sp.H = H; sp.d = d; sp.dp = dp; sp.map = map; sp.causal = causal;
        e = hh::launch_seq_f32(sp, (int)BH, s);
        if (e != hipSuccess) return hip_fail(e, "fp32 path launch");
        return ok();
    }

    float *wsS = nullptr, *wsZ = nullptr;
    if (pl.need_ws) {
        wsS = reinterpret_cast<float *>(workspace);
        wsZ = wsS + (size_t)BH * pl.nseg * pl.dpi * d;
    }
    const long slot_stride = pl.nseg;

    // Which state each segment starts from.
    const float *S_in = nullptr, *z_in = nullptr;
    long in_bh = 0, in_seg = 0;
    hh::PrefixParams pp;
    memset(&pp, 0, sizeof pp);
    pp.S_ws = wsS; pp.z_ws = wsZ; pp.S0 = S0; pp.z0 = z0;
    pp.BH = (int)BH; pp.nseg = pl.nseg; pp.dpi = pl.dpi; pp.dpc = dp; pp.d = d; pp.map = map;
    bool run_state = false, run_prefix = false;
    int state_segments = 0;
    if (causal) {
        if (pl.nseg > 1) {
            run_state = true;
            state_segments = pl.nseg - 1;
            run_prefix = true;
            pp.mode = 0;
            S_in = wsS; z_in = wsZ; in_bh = slot_stride; in_seg = 1;
        } else if (S0) {
            if (pl.narrow) {
                run_prefix = true;
                pp.mode = 0;
                S_in = wsS; z_in = wsZ; in_bh = 1; in_seg = 0;
            } else {
                S_in = S0; z_in = z0; in_bh = 1; in_seg = 0;
            }
        }
    } else {
        run_state = true;
        state_segments = pl.nseg;
        run_prefix = pl.nseg > 1;
        pp.mode = 1;
        pp.S0 = nullptr; pp.z0 = nullptr;
        S_in = wsS; z_in = wsZ; in_bh = slot_stride; in_seg = 0;
    }
    const int out_mode = causal ? 1 : 2;

    if (!pl.narrow) {
        // Segment slots: fp32 S in the kernels' register-image layout, fp32 z.  The scan between
        // the passes never sees S0; a caller's S0 is read directly by every segment.
        hh::WideParams wp;
        memset(&wp, 0, sizeof wp);
        wp.q = (const hh::bf16_t *)q; wp.k = (const hh::bf16_t *)k; wp.v = (const hh::bf16_t *)v;
        wp.W = (const hh::bf16_t *)W; wp.b = (const hh::bf16_t *)b; wp.y = (hh::bf16_t *)y;
        float *slS = nullptr;
        float *slZ = nullptr;
        if (pl.need_ws) {
            slS = reinterpret_cast<float *>(workspace);
            slZ = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + wide_slot_S_bytes(BH, pl.nseg, d));
        }
        wp.S_slots = slS; wp.z_slots = slZ; wp.slot_bh_stride = pl.nseg;
        wp.softmax = softmax_fused(map, dtype, causal, d) ? 1 : 0;
        // causal with few segments per sequence: the chunked pass sums the aggregates of the
        // earlier segments itself (at most 7 slots, still in L2) instead of a separate scan
        const bool direct_prefix = causal && pl.nseg <= 8;
        wp.N = N; wp.H = H; wp.BH = (int)BH; wp.seg_len = pl.seg_len;
        if (!causal && pl.nseg == 1 && d == 64) {
            // one segment per sequence: state and read-out in one workgroup, the total in LDS
            wp.nseg_grid = 1;
            e = hh::launch_bidir_fused(d, wp, (int)BH, s);
            if (e != hipSuccess) return hip_fail(e, "bidirectional forward launch");
            return ok();
        }
        if (run_state) {
            wp.nseg_grid = state_segments;
            e = hh::launch_wide(d, 0, wp, (int)(BH * state_segments), s);
            if (e != hipSuccess) return hip_fail(e, "segment-state launch");
            if (pl.nseg > 1 && !direct_prefix) {
                e = hh::launch_slot_scan(d, slS, slZ, (int)BH, pl.nseg, causal ? 0 : 1, s);
                if (e != hipSuccess) return hip_fail(e, "segment scan launch");
            }
        }
        if (causal) {
            wp.slot_mode = pl.nseg > 1 ? (direct_prefix ? 3 : 1) : 0;
            wp.S_in = S0; wp.z_in = z0; wp.in_bh_stride = 1; wp.in_seg_stride = 0;
        } else {
            wp.slot_mode = 2;
        }
        wp.S_out = S_out; wp.z_out = z_out;
        wp.nseg_grid = pl.nseg;
        e = hh::launch_wide(d, out_mode, wp, (int)(BH * pl.nseg), s);
        if (e != hipSuccess) return hip_fail(e, "chunked forward launch");
    } else {
        hh::NarrowParams np;
        memset(&np, 0, sizeof np);
        np.q = (const hh::bf16_t *)q; np.k = (const hh::bf16_t *)k; np.v = (const hh::bf16_t *)v;
        np.y = (hh::bf16_t *)y;
        np.S_ws = wsS; np.z_ws = wsZ; np.ws_bh_stride = slot_stride;
        np.coef = map == HH_MAP_QUADRATIC ? (const float *)W : nullptr;
        np.N = N; np.H = H; np.seg_len = pl.seg_len;
        if (run_state) {
            np.nseg_grid = state_segments;
            e = hh::launch_narrow(0, np, (int)(BH * state_segments), s);
            if (e != hipSuccess) return hip_fail(e, "segment-state launch");
        }
        if (run_prefix) {
            e = hh::launch_prefix(pp, s);
            if (e != hipSuccess) return hip_fail(e, "prefix launch");
        }
        np.S_in = S_in; np.z_in = z_in; np.in_bh_stride = in_bh; np.in_seg_stride = in_seg;
        np.S_out = S_out; np.z_out = z_out;
        np.S0c = S0; np.z0c = z0;
        np.nseg_grid = pl.nseg;
        e = hh::launch_narrow(out_mode, np, (int)(BH * pl.nseg), s);
        if (e != hipSuccess) return hip_fail(e, "chunked forward launch");
    }
    return ok();
}

hh_status_t hh_linattn_fwd_noalloc(int map, int dtype, int causal, int B, int H, int N, int d, const void *q,
                                   const void *k, const void *v, const void *W, const void *b, const float *S0,
                                   const float *z0, void *y, float *S_out, float *z_out, void *stream) {
    hh_status_t st = check_common(map, dtype, B, H, N, d);
    if (st != HH_OK) return st;
    if (causal != 0 && causal != 1) return fail(HH_EINVAL, "causal must be 0 or 1 (got %d)", causal);
    const size_t need = hh_linattn_fwd_workspace(map, dtype, causal, B, H, N, d);
    if (need > hh::kNoAllocScratchBytes)
        return fail(HH_EWORKSPACE,
                    "hh_linattn_fwd_noalloc: this problem needs %zu bytes of scratch, beyond the library's "
                    "fixed %zu; call hh_linattn_fwd with a workspace instead",
                    need, (size_t)hh::kNoAllocScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        clear_stale_hip_error();
        const hipError_t e = hh::noalloc_scratch(&ws);
        if (e != hipSuccess) return hip_fail(e, "scratch address");
    }
    return hh_linattn_fwd(map, dtype, causal, B, H, N, d, q, k, v, W, b, S0, z0, y, S_out, z_out, ws,
                          need > 0 ? hh::kNoAllocScratchBytes : 0, stream);
}

size_t hh_linattn_bwd_workspace(int map, int dtype, int causal, int B, int H, int N, int d) {
    if (check_common(map, dtype, B, H, N, d) != HH_OK || (causal != 0 && causal != 1) || dtype != HH_BF16 ||
        quadratic_family(map) || N == 0)
        return 0;
    return make_bwd_plan(map, (long)B * H, N, d).bytes;
}

hh_status_t hh_linattn_bwd(int map, int dtype, int causal, int B, int H, int N, int d, const void *q, const void *k,
                           const void *v, const void *W, const void *b, const void *y, const void *dy, void *dq,
                           void *dk, void *dv, float *dW, float *db, void *workspace, size_t workspace_bytes,
                           void *stream) {
    hh_status_t st = check_common(map, dtype, B, H, N, d);
    if (st != HH_OK) return st;
    if (causal != 0 && causal != 1) return fail(HH_EINVAL, "causal must be 0 or 1 (got %d)", causal);
    if (dtype != HH_BF16) return fail(HH_EUNSUPPORTED, "backward: bf16 inputs only");
    if (quadratic_family(map)) return fail(HH_EUNSUPPORTED, "backward: the exponential and softmax maps only");
    const bool need = N > 0;
    const char *names[9] = {"q", "k", "v", "y", "dy", "dq", "dk", "dv", "dW"};
    const void *ptrs[9] = {q, k, v, y, dy, dq, dk, dv, dW};
    for (int i = 0; i < 9; i++)
        if ((st = check_ptr(ptrs[i], names[i], need || i == 8)) != HH_OK) return st;
    if ((st = check_params(map, W, b, true)) != HH_OK) return st;
    if ((st = check_ptr(db, "db", false)) != HH_OK) return st;
    if (map_has_b(map) ? (b != nullptr) != (db != nullptr) : db != nullptr)
        return fail(HH_EINVAL, "db must be given exactly when the map has a bias and b is given");
    const long BH = (long)B * H;
    const size_t nio = (size_t)BH * N * d * 2, nW = (size_t)H * d * d * 4, nb = (size_t)H * d * 4;
    const void *ins[6] = {q, k, v, y, dy, W};
    void *outs[3] = {dq, dk, dv};
    for (int o = 0; o < 3; o++) {
        for (int i = 0; i < 6; i++)
            if (overlap(outs[o], nio, ins[i], i == 5 ? (size_t)H * d * d * 2 : nio))
                return fail(HH_EINVAL, "an input gradient overlaps an input");
        for (int o2 = o + 1; o2 < 3; o2++)
            if (overlap(outs[o], nio, outs[o2], nio)) return fail(HH_EINVAL, "input gradients overlap");
        if (overlap(outs[o], nio, dW, nW) || overlap(outs[o], nio, db, nb)) return fail(HH_EINVAL, "gradients overlap");
    }
    if (overlap(dW, nW, db, nb)) return fail(HH_EINVAL, "dW overlaps db");
    const BwdPlan pl = make_bwd_plan(map, BH, N, d);
    if (N > 0) {
        if (!workspace) return fail(HH_EWORKSPACE, "workspace of %zu bytes required, got NULL", pl.bytes);
        if (workspace_bytes < pl.bytes)
            return fail(HH_EWORKSPACE, "workspace of %zu bytes required, got %zu", pl.bytes, workspace_bytes);
        if (!aligned16(workspace)) return fail(HH_EINVAL, "workspace is not 16-byte aligned");
        for (int i = 0; i < 6; i++)
            if (overlap(workspace, pl.bytes, ins[i], i == 5 ? (size_t)H * d * d * 2 : nio))
                return fail(HH_EINVAL, "workspace overlaps an input");
        for (int o = 0; o < 3; o++)
            if (overlap(workspace, pl.bytes, outs[o], nio)) return fail(HH_EINVAL, "workspace overlaps an output");
        if (overlap(workspace, pl.bytes, dW, nW) || overlap(workspace, pl.bytes, db, nb))
            return fail(HH_EINVAL, "workspace overlaps an output");
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    clear_stale_hip_error();
    hipError_t e;
    if (N == 0) {  // no tokens: the parameter gradients are zero
        e = hh::launch_state_copy(nullptr, nullptr, dW, db ? db : dW, (long)H * d * d, db ? (long)H * d : 0, s);
        if (e != hipSuccess) return hip_fail(e, "zero gradients launch");
        return ok();
    }
    char *ws = reinterpret_cast<char *>(workspace);
    hh::bf16_t *phiq = reinterpret_cast<hh::bf16_t *>(ws), *phik = reinterpret_cast<hh::bf16_t *>(ws + pl.off_phik);
    // features of q and k (bf16, as the forward's matrix cores take them)
    if (map == HH_MAP_HEDGEHOG) {
        e = hh::launch_featuremap_hedgehog_bf16(d, (const hh::bf16_t *)q, (const hh::bf16_t *)W, (const hh::bf16_t *)b,
                                                phiq, (int)BH, H, N, s);
        if (e == hipSuccess)
            e = hh::launch_featuremap_hedgehog_bf16(d, (const hh::bf16_t *)k, (const hh::bf16_t *)W,
                                                    (const hh::bf16_t *)b, phik, (int)BH, H, N, s);
    } else {
        e = hh::launch_featuremap_variant(map, dtype, d, q, W, b, phiq, BH, H, N, s);
        if (e == hipSuccess) e = hh::launch_featuremap_variant(map, dtype, d, k, W, b, phik, BH, H, N, s);
    }
    if (e != hipSuccess) return hip_fail(e, "feature map launch");
    float *Ssl = reinterpret_cast<float *>(ws + pl.off_S), *zsl = reinterpret_cast<float *>(ws + pl.off_z);
    float *Rsl = reinterpret_cast<float *>(ws + pl.off_R), *rsl = reinterpret_cast<float *>(ws + pl.off_r);
    // forward sums per segment (canonical), scanned into exclusive prefixes (causal) or the total
    hh::FeatParams fp;
    memset(&fp, 0, sizeof fp);
    fp.phiq = phiq; fp.phik = phik; fp.v = (const hh::bf16_t *)v;
    fp.S_slots = Ssl; fp.z_slots = zsl; fp.slot_bh_stride = pl.nseg; fp.slot_canonical = 1;
    fp.N = N; fp.seg_len = pl.seg_len;
    const int nstate = causal ? pl.nseg - 1 : pl.nseg;
    if (nstate > 0) {
        fp.nseg_grid = nstate;
        e = hh::launch_feat(d, pl.dp, 0, fp, (int)(BH * nstate), s);
        if (e == hipSuccess && pl.nseg > 1) e = hh::launch_feat_scan(Ssl, zsl, d, pl.dp, (int)BH, pl.nseg, causal ? 0 : 1, s);
        if (e != hipSuccess) return hip_fail(e, "forward sums launch");
    }
    hh::BwdParams bp;
    memset(&bp, 0, sizeof bp);
    bp.phiq = phiq; bp.phik = phik; bp.v = (const hh::bf16_t *)v; bp.y = (const hh::bf16_t *)y;
    bp.dy = (const hh::bf16_t *)dy; bp.q = (const hh::bf16_t *)q; bp.k = (const hh::bf16_t *)k;
    bp.W = (const hh::bf16_t *)W; bp.b = map_has_b(map) ? (const hh::bf16_t *)b : nullptr;
    bp.dphiq = reinterpret_cast<hh::bf16_t *>(ws + pl.off_dphiq); bp.dphik = reinterpret_cast<hh::bf16_t *>(ws + pl.off_dphik);
    bp.den_c = reinterpret_cast<float *>(ws + pl.off_denc);
    bp.S_slots = Ssl; bp.z_slots = zsl; bp.R_slots = Rsl; bp.r_slots = rsl;
    bp.dq = (hh::bf16_t *)dq; bp.dk = (hh::bf16_t *)dk; bp.dv = (hh::bf16_t *)dv;
    bp.dW_parts = reinterpret_cast<float *>(ws + pl.off_parts);
    bp.N = N; bp.H = H; bp.nseg = pl.nseg; bp.seg_len = pl.seg_len;
    e = hh::launch_bwd_pass(0, d, pl.dp, causal, bp, (int)(BH * pl.nseg), s);
    if (e != hipSuccess) return hip_fail(e, "q-side backward launch");
    if (pl.nseg > 1) {
        e = hh::launch_feat_scan(Rsl, rsl, d, pl.dp, (int)BH, pl.nseg, causal ? 0 : 1, s);
        if (e != hipSuccess) return hip_fail(e, "reverse sums launch");
    }
    e = hh::launch_bwd_pass(1, d, pl.dp, causal, bp, (int)(BH * pl.nseg), s);
    if (e != hipSuccess) return hip_fail(e, "k-side backward launch");
    e = hh::launch_bwd_map(map, d, bp, BH, s);
    if (e == hipSuccess) e = hh::launch_bwd_reduce(bp.dW_parts, dW, db, B, H, d, N, s);
    if (e != hipSuccess) return hip_fail(e, "feature-map backward launch");
    return ok();
}

size_t hh_distill_loss_workspace(int map, int dtype, int B, int H, int N, int d) {
    if (check_common(map, dtype, B, H, N, d) != HH_OK || dtype != HH_BF16 || map != HH_MAP_HEDGEHOG) return 0;
    return (size_t)B * H * N * 2 * d * sizeof(uint16_t);  // the features of k
}

hh_status_t hh_distill_loss(int map, int dtype, int B, int H, int N, int d, const void *q, const void *k,
                            const void *W, const void *b, float *loss, void *workspace, size_t workspace_bytes,
                            void *stream) {
    hh_status_t st = check_common(map, dtype, B, H, N, d);
    if (st != HH_OK) return st;
    if (dtype != HH_BF16) return fail(HH_EUNSUPPORTED, "distillation loss: bf16 inputs only");
    if (map != HH_MAP_HEDGEHOG && map != HH_MAP_TAYLOR2)
        return fail(HH_EUNSUPPORTED, "distillation loss: the Hedgehog and Taylor maps only");
    const bool hog = map == HH_MAP_HEDGEHOG;
    const bool need = N > 0;
    if ((st = check_ptr(q, "q", need)) != HH_OK) return st;
    if ((st = check_ptr(k, "k", need)) != HH_OK) return st;
    if ((st = check_ptr(loss, "loss", need)) != HH_OK) return st;
    if (hog) {
        if ((st = check_ptr(W, "W", need)) != HH_OK) return st;
        if ((st = check_ptr(b, "b", false)) != HH_OK) return st;
    }
    const long BH = (long)B * H;
    const size_t nio = (size_t)BH * N * d * sizeof(uint16_t), nl = (size_t)BH * N * sizeof(float);
    if (overlap(loss, nl, q, nio) || overlap(loss, nl, k, nio)) return fail(HH_EINVAL, "loss overlaps q or k");
    const size_t need_ws = hh_distill_loss_workspace(map, dtype, B, H, N, d);
    if (need_ws > 0) {
        if (!workspace) return fail(HH_EWORKSPACE, "workspace of %zu bytes required, got NULL", need_ws);
        if (workspace_bytes < need_ws)
            return fail(HH_EWORKSPACE, "workspace of %zu bytes required, got %zu", need_ws, workspace_bytes);
        if (!aligned16(workspace)) return fail(HH_EINVAL, "workspace is not 16-byte aligned");
        if (overlap(workspace, need_ws, q, nio) || overlap(workspace, need_ws, k, nio) ||
            overlap(workspace, need_ws, loss, nl))
            return fail(HH_EINVAL, "workspace overlaps an input or output");
    }
    if (N == 0) return ok();
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    clear_stale_hip_error();
    hipError_t e;
    hh::DistillParams dp;
    dp.q = (const hh::bf16_t *)q; dp.k = (const hh::bf16_t *)k;
    dp.phi_k = nullptr;
    dp.W = hog ? (const hh::bf16_t *)W : nullptr;
    dp.b = hog ? (const hh::bf16_t *)b : nullptr;
    dp.loss = loss; dp.N = N; dp.BH = (int)BH; dp.H = H;
    if (hog) {
        hh::bf16_t *fk = reinterpret_cast<hh::bf16_t *>(workspace);
        e = hh::launch_featuremap_hedgehog_bf16(d, (const hh::bf16_t *)k, (const hh::bf16_t *)W,
                                                (const hh::bf16_t *)b, fk, (int)BH, H, N, s);
        if (e != hipSuccess) return hip_fail(e, "feature map launch");
        dp.phi_k = fk;
    }
    e = hh::launch_distill(map, d, dp, (int)BH, s);
    if (e != hipSuccess) return hip_fail(e, "distillation loss launch");
    return ok();
}

hh_status_t hh_linattn_decode_step(int map, int dtype, int B, int H, int d, const void *q, const void *k,
                                   const void *v, const void *W, const void *b, float *S, float *z, void *y,
                                   void *stream) {
    hh_status_t st = check_common(map, dtype, B, H, 1, d);
    if (st != HH_OK) return st;
    const int dp = feature_dim(map, d);
    const long BH = (long)B * H;
    const size_t eb = elem_bytes(dtype);
    if ((st = check_ptr(q, "q", true)) != HH_OK) return st;
    if ((st = check_ptr(k, "k", true)) != HH_OK) return st;
    if ((st = check_ptr(v, "v", true)) != HH_OK) return st;
    if ((st = check_ptr(y, "y", true)) != HH_OK) return st;
    if ((st = check_ptr(S, "S", true)) != HH_OK) return st;
    if ((st = check_ptr(z, "z", true)) != HH_OK) return st;
    if ((st = check_params(map, W, b, true)) != HH_OK) return st;
    const size_t nio = (size_t)BH * d * eb;
    const size_t nS = (size_t)BH * dp * d * sizeof(float), nz = (size_t)BH * dp * sizeof(float);
    if (overlap(y, nio, q, nio) || overlap(y, nio, k, nio) || overlap(y, nio, v, nio) || overlap(y, nio, S, nS) ||
        overlap(y, nio, z, nz))
        return fail(HH_EINVAL, "y overlaps q, k, v, S or z");
    if (overlap(S, nS, z, nz)) return fail(HH_EINVAL, "S overlaps z");
    hh::DecodeParams dpar;
    dpar.q = q; dpar.k = k; dpar.v = v; dpar.W = map_has_W(map) ? W : nullptr; dpar.b = map_has_b(map) ? b : nullptr;
    dpar.y = y; dpar.S = S; dpar.z = z;
    dpar.H = H; dpar.d = d; dpar.dp = dp; dpar.map = map; dpar.dtype = dtype;
    clear_stale_hip_error();
    hipError_t e = hh::launch_decode(dpar, (int)BH, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return ok();
}

}  // extern "C"
