// hh_bwd.hip -- backward of the linear-attention forward: gradients of a loss L with respect
// to q, k, v and the feature map's W and b, given dL/dy (what training from scratch needs: the
// walkthrough's section 3.4, "Training Protocols for the Three Regimes").
//
// With phi_q(i) = phi(q_i), phi_k(j) = phi(k_j), den_i = sum_{j visible} phi_q(i).phi_k(j) and
// y_i = sum_j phi_q(i).phi_k(j) v_j / den_i (Eq. 2), write g_i = dy_i / den_i and
// c_i = -(dy_i . y_i) / den_i.  Then, with visibility j <= i (causal) or all j:
//     dL/dphi_q(i) = S_i g_i + c_i z_i                  S_i = sum_{j vis} phi_k(j) v_j^T, z_i = sum phi_k(j)
//     dL/dphi_k(j) = R_j v_j + r_j                      R_j = sum_{i: j vis} phi_q(i) g_i^T, r_j = sum c_i phi_q(i)
//     dL/dv_j      = R_j^T phi_k(j)
// and dL/dq, dL/dk, dL/dW, dL/db follow from dL/dphi by the chain rule through the map.
// Per 64-token chunk c (causal), with the running sums before (S, z) or after (R, r) the chunk
// and M_c = tril(G_c V_c^T + c_c 1^T), P_c = tril(phiQ_c phiK_c^T):
//     dphiQ_c = G_c S^T + c_c z^T + M_c phiK_c                    (chunks in order)
//     dphiK_c = V_c R^T + 1 r^T + M_c^T phiQ_c,   dV_c = phiK_c R + P_c^T G_c   (chunks in reverse)
// The same regrouping as the forward's chunks (only rounding differs).  Kernels:
//   bwd_q_kernel   per segment, chunks in order: den and c per token, dphiQ (bf16), and the
//                  segment's reverse-sum aggregate (R, r) for the k side;
//   bwd_k_kernel   per segment, chunks in reverse: dphiK (bf16) and dV;
//   bwd_map_kernel per 64 tokens: u recomputed, dL/du from dL/dphi, dx = W^T du, and this
//                  workgroup's part of dW = sum du x^T and db = sum du;
//   bwd_reduce_kernel: the parts of dW and db summed per head.
// The forward sums S, z per segment come from the features-given state pass (hh_feat.hip),
// scanned into exclusive prefixes; the reverse sums likewise, the segments taken in reverse.
#include "hh_common.h"
#include "hh_kernels.h"

namespace hh {

namespace {

enum { BW_CAUSAL = 1, BW_BIDIR = 0 };

typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 tr_read(const bf16_t *p) {
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t *)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// MFMA operand whose K index runs down the rows of a row-major LDS tile: lane (g, r16) gets
// column c0 + r16 and rows r0 + 8 g .. r0 + 8 g + 7 (lane_off = (8 g + r16 / 4) pitch + 4 (r16 % 4)).
__device__ __forceinline__ bf16x8 down_rows(const bf16_t *tile, int lane_off, int r0, int c0, int pitch) {
    const bf16_t *p = tile + lane_off + r0 * pitch + c0;
    return cat(tr_read(p), tr_read(p + 4 * pitch));
}
// The same with the K order of two stacked accumulator blocks: rows r0 + 4 g .. + 3, then
// r0 + 16 + 4 g .. + 3 (lane_off_p = (4 g + r16 / 4) pitch + 4 (r16 % 4)).
__device__ __forceinline__ bf16x8 down_rows_perm(const bf16_t *tile, int lane_off_p, int r0, int c0, int pitch) {
    const bf16_t *p = tile + lane_off_p + r0 * pitch + c0;
    return cat(tr_read(p), tr_read(p + 16 * pitch));
}
// Row operand in the permuted K order: elements k0 + 4 g .. + 3 and k0 + 16 + 4 g .. + 3 of a row.
__device__ __forceinline__ bf16x8 row_perm(const bf16_t *row, int k0, int g) {
    return cat(load4(row + k0 + 4 * g), load4(row + k0 + 16 + 4 * g));
}

constexpr int pitch_of(int n) { return n + (((16 - n) % 64) + 64) % 64; }

template <int D, int DP>
struct BwdCfg {
    static constexpr int C = 64;
    static constexpr int NW = D / 16;                 // waves
    static constexpr int NT = 64 * NW;
    static constexpr int DPP = (DP + 31) / 32 * 32;   // features padded to whole K steps
    static constexpr int DVP = (D + 31) / 32 * 32;    // value columns padded likewise
    static constexpr int FB = DPP / 16, VB = D / 16, VBP = DVP / 16;
    static constexpr int FBW = FB / NW;               // feature blocks per wave (1 or 2)
    static constexpr int KSF = DPP / 32, KSV = DVP / 32;
    static constexpr int PF = pitch_of(DPP), PV = pitch_of(DVP), PM = pitch_of(C);
    static constexpr int SZ_F = C * PF * 2, SZ_V = C * PV * 2, SZ_M = C * PM * 2;
    static constexpr int OFF_Q = 0, OFF_K = SZ_F, OFF_V = 2 * SZ_F, OFF_G = OFF_V + SZ_V;
    static constexpr int OFF_DY = OFF_G + SZ_V;
    static constexpr int OFF_M = OFF_DY + SZ_V, OFF_P = OFF_M + SZ_M;
    static constexpr int OFF_F32 = OFF_P + SZ_M;     // fp32 arrays below
    // den partials [NW][C], row sums [4][C], den [C], c [C], z or r per feature [DPP]
    static constexpr int F32_WORDS = (NW + 4) * C + 2 * C + DPP;
    static constexpr int LDS_BYTES = OFF_F32 + 4 * F32_WORDS;
    static constexpr int PQ = C * DP / 8 / NT, PVV = C * D / 8 / NT;
    static_assert(FBW == 1 || FBW == 2, "feature blocks split evenly over the waves");
    static_assert(PQ * NT * 8 == C * DP && PVV * NT * 8 == C * D, "whole pieces per thread");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// (a uniform base plus the piece's 32-bit element offset: 64-bit per-piece addresses would be
// kept live across the chunk loop and spill)
template <int n>
__device__ __forceinline__ bf16x8 load_piece(const bf16_t *src, int p, int valid) {
    const int row = p / (n / 8), col = 8 * (p % (n / 8));
    return row < valid ? *reinterpret_cast<const bf16x8 *>(src + (uint32_t)(row * n + col)) : zero_bf16x8();
}
template <int n, int pitch>
__device__ __forceinline__ void store_piece(bf16_t *tile, int p, const bf16x8 &x) {
    const int row = p / (n / 8), col = 8 * (p % (n / 8));
    *reinterpret_cast<bf16x8 *>(tile + row * pitch + col) = x;
}

// Stage one chunk (rows >= valid zero): phi(q), phi(k), v, dy, and with WITH_Y also y (into
// the tile that holds G later).  PERM_KV: phi(k) and v in the reordered column order of
// qperm_pos (the k side, whose products take their rows in accumulator-pair K order).
template <int D, int DP, bool WITH_Y = false, bool PERM_KV = false>
__device__ __forceinline__ void bwd_stage(const BwdParams &p, size_t tok0, int valid, unsigned char *smem, int tid) {
    using K = BwdCfg<D, DP>;
    bf16_t *sQ = reinterpret_cast<bf16_t *>(smem + K::OFF_Q), *sK = reinterpret_cast<bf16_t *>(smem + K::OFF_K);
    bf16_t *sV = reinterpret_cast<bf16_t *>(smem + K::OFF_V), *sDY = reinterpret_cast<bf16_t *>(smem + K::OFF_DY);
    bf16x8 a[K::PQ], bq[K::PQ], c[K::PVV], e[K::PVV], yv[K::PVV];
    // the piece offsets are recomputed per chunk from an opaque copy of the thread index: kept
    // live across the chunk loop instead, they push the q-side kernel into spills
    asm volatile("" : "+v"(tid));
#pragma unroll
    for (int i = 0; i < K::PQ; i++) {
        a[i] = load_piece<DP>(p.phiq + tok0 * DP, tid + K::NT * i, valid);
        bq[i] = load_piece<DP>(p.phik + tok0 * DP, tid + K::NT * i, valid);
    }
#pragma unroll
    for (int i = 0; i < K::PVV; i++) {
        c[i] = load_piece<D>(p.v + tok0 * D, tid + K::NT * i, valid);
        e[i] = load_piece<D>(p.dy + tok0 * D, tid + K::NT * i, valid);
        if (WITH_Y) yv[i] = load_piece<D>(p.y + tok0 * D, tid + K::NT * i, valid);
    }
    if (WITH_Y) {
        bf16_t *sY = reinterpret_cast<bf16_t *>(smem + K::OFF_G);
#pragma unroll
        for (int i = 0; i < K::PVV; i++) store_piece<D, K::PV>(sY, tid + K::NT * i, yv[i]);
    }
#pragma unroll
    for (int i = 0; i < K::PQ; i++) {
        store_piece<DP, K::PF>(sQ, tid + K::NT * i, a[i]);
        const int pe = tid + K::NT * i;
        if (PERM_KV) store8_qperm(sK + (pe / (DP / 8)) * K::PF, 8 * (pe % (DP / 8)), bq[i]);
        else store_piece<DP, K::PF>(sK, pe, bq[i]);
    }
#pragma unroll
    for (int i = 0; i < K::PVV; i++) {
        const int pe = tid + K::NT * i;
        if (PERM_KV) store8_qperm(sV + (pe / (D / 8)) * K::PV, 8 * (pe % (D / 8)), c[i]);
        else store_piece<D, K::PV>(sV, pe, c[i]);
        store_piece<D, K::PV>(sDY, tid + K::NT * i, e[i]);
    }
}

__device__ __forceinline__ void head_segment(int nseg, int &bh, int &s) {
    const int b = blockIdx.x, BH = gridDim.x / nseg;
    if (BH % 8 == 0) {
        const int j = b >> 3;
        bh = (b & 7) + 8 * (j / nseg);
        s = j % nseg;
    } else {
        bh = b / nseg;
        s = b % nseg;
    }
}

// Scores of one chunk into an LDS tile [query][key] (bf16, keys after the query zeroed when
// causal) and their row sums; blocks dealt over the waves.
template <int D, int DP, int MODE>
__device__ __forceinline__ void bwd_scores(const bf16_t *sQ, const bf16_t *sK, bf16_t *sP, float *sRS, int w, int g,
                                           int r16) {
    using K = BwdCfg<D, DP>;
    const int nblk = MODE == BW_CAUSAL ? 10 : 16;
    for (int t = w; t < nblk; t += K::NW) {
        int ib, jb;
        if (MODE == BW_CAUSAL) {
            ib = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
            jb = t - ib * (ib + 1) / 2;
        } else {
            ib = t >> 2;
            jb = t & 3;
        }
        f32x4 a = zero4();
#pragma unroll
        for (int ks = 0; ks < K::KSF; ks++)
            a = mfma_bf16(*reinterpret_cast<const bf16x8 *>(sK + (16 * jb + r16) * K::PF + 32 * ks + 8 * g),
                          *reinterpret_cast<const bf16x8 *>(sQ + (16 * ib + r16) * K::PF + 32 * ks + 8 * g), a);
        if (MODE == BW_CAUSAL && jb == ib) {
#pragma unroll
            for (int r = 0; r < 4; r++)
                if (4 * g + r > r16) a[r] = 0.0f;
        }
        const bf16x4 ab = to_bf16x4(a);
        store4(sP + (16 * ib + r16) * K::PM + 16 * jb + 4 * g, ab);
        float rs = ((float)ab[0] + (float)ab[1]) + ((float)ab[2] + (float)ab[3]);
        rs += __shfl_xor(rs, 16);
        rs += __shfl_xor(rs, 32);
        if (g == 0) sRS[jb * K::C + 16 * ib + r16] = rs;
    }
}

// M = G V^T + c 1^T (keys after the query zeroed when causal) into an LDS tile [query][key].
// G is held in the reordered column order of qperm_pos, V in the natural one.
template <int D, int DP, int MODE>
__device__ __forceinline__ void bwd_mtile(const bf16_t *sG, const bf16_t *sV, const float *sC, bf16_t *sM, int w,
                                          int g, int r16) {
    using K = BwdCfg<D, DP>;
    const int nblk = MODE == BW_CAUSAL ? 10 : 16;
    for (int t = w; t < nblk; t += K::NW) {
        int ib, jb;
        if (MODE == BW_CAUSAL) {
            ib = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
            jb = t - ib * (ib + 1) / 2;
        } else {
            ib = t >> 2;
            jb = t & 3;
        }
        // out[key][query]: A = V rows (keys), B = G rows (queries), K = value columns
        f32x4 a = zero4();
#pragma unroll
        for (int ks = 0; ks < K::KSV; ks++)
            a = mfma_bf16(row_perm(sV + (16 * jb + r16) * K::PV, 32 * ks, g),
                          *reinterpret_cast<const bf16x8 *>(sG + (16 * ib + r16) * K::PV + 32 * ks + 8 * g), a);
        const float ci = sC[16 * ib + r16];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            a[r] += ci;
            if (MODE == BW_CAUSAL && jb == ib && 4 * g + r > r16) a[r] = 0.0f;
        }
        store4(sM + (16 * ib + r16) * K::PM + 16 * jb + 4 * g, to_bf16x4(a));
    }
}

// The k side's tiles stored transposed, [key][query] (the operands swapped in the product), so
// that its products read them as plain 16-byte rows: read down the rows of a 64-column tile
// (128-byte rows) the transposing reads conflict in the LDS banks.  Scores without row sums.
// phi(k) and V are held in the reordered column order (bwd_stage with PERM_KV), so their rows
// are 16-byte reads here and phi(q), G are read in the matching order.
template <int D, int DP, int MODE>
__device__ __forceinline__ void bwd_scores_t(const bf16_t *sQ, const bf16_t *sK, bf16_t *sPT, int w, int g, int r16) {
    using K = BwdCfg<D, DP>;
    const int nblk = MODE == BW_CAUSAL ? 10 : 16;
    for (int t = w; t < nblk; t += K::NW) {
        int ib, jb;
        if (MODE == BW_CAUSAL) {
            ib = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
            jb = t - ib * (ib + 1) / 2;
        } else {
            ib = t >> 2;
            jb = t & 3;
        }
        // lane: key 16 jb + r16, queries 16 ib + 4 g + r; keep key <= query
        f32x4 a = zero4();
#pragma unroll
        for (int ks = 0; ks < K::KSF; ks++)
            a = mfma_bf16(row_perm(sQ + (16 * ib + r16) * K::PF, 32 * ks, g),
                          *reinterpret_cast<const bf16x8 *>(sK + (16 * jb + r16) * K::PF + 32 * ks + 8 * g), a);
        if (MODE == BW_CAUSAL && jb == ib) {
#pragma unroll
            for (int r = 0; r < 4; r++)
                if (4 * g + r < r16) a[r] = 0.0f;
        }
        store4(sPT + (16 * jb + r16) * K::PM + 16 * ib + 4 * g, to_bf16x4(a));
    }
}

template <int D, int DP, int MODE>
__device__ __forceinline__ void bwd_mtile_t(const bf16_t *sG, const bf16_t *sV, const float *sC, bf16_t *sMT, int w,
                                            int g, int r16) {
    using K = BwdCfg<D, DP>;
    const int nblk = MODE == BW_CAUSAL ? 10 : 16;
    for (int t = w; t < nblk; t += K::NW) {
        int ib, jb;
        if (MODE == BW_CAUSAL) {
            ib = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
            jb = t - ib * (ib + 1) / 2;
        } else {
            ib = t >> 2;
            jb = t & 3;
        }
        // lane: key 16 jb + r16, queries 16 ib + 4 g + r
        f32x4 a = zero4();
#pragma unroll
        for (int ks = 0; ks < K::KSV; ks++)
            a = mfma_bf16(row_perm(sG + (16 * ib + r16) * K::PV, 32 * ks, g),
                          *reinterpret_cast<const bf16x8 *>(sV + (16 * jb + r16) * K::PV + 32 * ks + 8 * g), a);
        const f32x4 cq = *reinterpret_cast<const f32x4 *>(sC + 16 * ib + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; r++) {
            a[r] += cq[r];
            if (MODE == BW_CAUSAL && jb == ib && 4 * g + r < r16) a[r] = 0.0f;
        }
        store4(sMT + (16 * jb + r16) * K::PM + 16 * ib + 4 * g, to_bf16x4(a));
    }
}

// ---- q side -----------------------------------------------------------------------------
template <int D, int DP, int MODE>
__device__ void bwd_q_body(const BwdParams &p, unsigned char *smem, int bh, int s) {
    using K = BwdCfg<D, DP>;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int t_begin = s * p.seg_len, t_end = min(p.N, t_begin + p.seg_len);
    const int n = (t_end - t_begin + K::C - 1) / K::C;
    const size_t tok_base = (size_t)bh * p.N;
    bf16_t *sQ = reinterpret_cast<bf16_t *>(smem + K::OFF_Q), *sK = reinterpret_cast<bf16_t *>(smem + K::OFF_K);
    bf16_t *sV = reinterpret_cast<bf16_t *>(smem + K::OFF_V), *sG = reinterpret_cast<bf16_t *>(smem + K::OFF_G);
    bf16_t *sDY = reinterpret_cast<bf16_t *>(smem + K::OFF_DY);
    bf16_t *sM = reinterpret_cast<bf16_t *>(smem + K::OFF_M), *sP = reinterpret_cast<bf16_t *>(smem + K::OFF_P);
    float *sDen = reinterpret_cast<float *>(smem + K::OFF_F32);   // [NW][C]
    float *sRS = sDen + K::NW * K::C;                              // [4][C]
    float *sDn = sRS + 4 * K::C, *sC = sDn + K::C;                 // den, c per query
    float *sZ = sC + K::C;                                         // z per feature (before the chunk)

    for (int i = tid; i < K::LDS_BYTES / 16; i += K::NT) reinterpret_cast<f32x4 *>(smem)[i] = zero4();
    __syncthreads();

    // S^T by features: ST[vb][j] rows value columns 16 vb + 4 g + r, column feature 16 (FBW w + j) + r16
    f32x4 ST[K::VB][K::FBW];
    // R by value columns (this segment's reverse-sum aggregate): rows features 16 fb + 4 g + r,
    // column value 16 w + r16; r by features: every row the same
    f32x4 Racc[K::FB], racc[K::FBW];
#pragma unroll
    for (int vb = 0; vb < K::VB; vb++)
#pragma unroll
        for (int j = 0; j < K::FBW; j++) ST[vb][j] = zero4();
#pragma unroll
    for (int fb = 0; fb < K::FB; fb++) Racc[fb] = zero4();
#pragma unroll
    for (int j = 0; j < K::FBW; j++) racc[j] = zero4();
    // starting sums: exclusive prefix (causal, slot s) or the total (bidirectional, slot 0), canonical
    {
        const long sl = MODE == BW_CAUSAL ? (s > 0 ? (long)bh * p.nseg + s : -1) : (long)bh * p.nseg;
        if (sl >= 0) {
            const float *Sp = p.S_slots + sl * (long)K::DPP * D;
            const float *zp = p.z_slots + sl * (long)K::DPP;
#pragma unroll
            for (int vb = 0; vb < K::VB; vb++)
#pragma unroll
                for (int j = 0; j < K::FBW; j++) {
                    const int f = 16 * (K::FBW * w + j) + r16;
                    ST[vb][j] = *reinterpret_cast<const f32x4 *>(Sp + (size_t)f * D + 16 * vb + 4 * g);
                }
            for (int f = tid; f < K::DPP; f += K::NT) sZ[f] = zp[f];
        }
    }
    __syncthreads();

    const int lo = 4 * (r16 & 3), lr = 8 * g + (r16 >> 2);  // transposing-read lane offsets (column, row)
    const bf16x8 ones = ones_bf16x8();
    // dy . y of query i is summed by the TPQ = D / 16 threads TPQ i .. TPQ i + TPQ - 1, each over
    // 16 columns; y is staged with the chunk (in the G tile, free until G is formed), so that its
    // loads share the chunk's one memory wait
    constexpr int TPQ = K::NT / K::C;
    static_assert(TPQ * K::C == K::NT && TPQ * 16 == D, "whole 16-column parts per thread");
    const int yi = tid / TPQ, ypart = tid % TPQ;
    for (int c = 0; c < n; c++) {
        const int t0 = t_begin + K::C * c;
        const int valid = min(K::C, t_end - t0);
        bwd_stage<D, DP, true>(p, tok_base + t0, valid, smem, tid);
        __syncthreads();
        // ---- den: phi_q . z (partials per wave over its features) + intra row sums
        if (MODE == BW_CAUSAL) bwd_scores<D, DP, MODE>(sQ, sK, sP, sRS, w, g, r16);
        {
            // z of this wave's features as an A operand (every row the same), K = features
            const float *zb = sZ + 32 * w * K::FBW / 2;  // FBW = 2: features 32 w ..; FBW = 1: 16 w ..
#pragma unroll
            for (int ib = 0; ib < 4; ib++) {
                f32x4 dacc = zero4();
                if (K::FBW == 2) {
                    bf16x8 za;
#pragma unroll
                    for (int e2 = 0; e2 < 8; e2++) za[e2] = (__bf16)zb[8 * g + e2];
                    dacc = mfma_bf16(za, *reinterpret_cast<const bf16x8 *>(sQ + (16 * ib + r16) * K::PF + 32 * w + 8 * g),
                                     dacc);
                } else {
                    // one block of 16 features 16 w ..: the K step 32 (w / 2) with the other half zero
                    bf16x8 za;
#pragma unroll
                    for (int e2 = 0; e2 < 8; e2++) {
                        const int f = 32 * (w >> 1) + 8 * g + e2;
                        za[e2] = (f >> 4) == w ? (__bf16)sZ[f] : (__bf16)0.0f;
                    }
                    dacc = mfma_bf16(za, *reinterpret_cast<const bf16x8 *>(sQ + (16 * ib + r16) * K::PF + 32 * (w >> 1) + 8 * g),
                                     dacc);
                }
                if (g == 0) sDen[w * K::C + 16 * ib + r16] = dacc[0];
            }
        }
        __syncthreads();
        // ---- den, g = dy / den, c = -(dy . y) / den (queries past the end: 0)
        {
            float dot = 0.0f;
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int col = 16 * ypart + 8 * j;
                const bf16x8 yv = *reinterpret_cast<const bf16x8 *>(sG + yi * K::PV + col);
                const bf16x8 dv = *reinterpret_cast<const bf16x8 *>(sDY + yi * K::PV + col);
#pragma unroll
                for (int e2 = 0; e2 < 8; e2++) dot = fmaf((float)dv[e2], (float)yv[e2], dot);
            }
#pragma unroll
            for (int o = 1; o < TPQ; o <<= 1) dot += __shfl_xor(dot, o);
            if (ypart == 0) {
            const int i = yi;
            float den = 0.0f;
#pragma unroll
            for (int pw = 0; pw < K::NW; pw++) den += sDen[pw * K::C + i];
            if (MODE == BW_CAUSAL) {
#pragma unroll
                for (int jb = 0; jb < 4; jb++) den += sRS[jb * K::C + i];
            }
            const bool live = i < valid;
            const float rd = live ? 1.0f / den : 0.0f;
            sDn[i] = rd;
            sC[i] = live ? -dot * rd : 0.0f;
            if (live) {
                p.den_c[2 * (tok_base + t0 + i)] = den;
                p.den_c[2 * (tok_base + t0 + i) + 1] = -dot * rd;
            }
            }
        }
        __syncthreads();
        // G in the reordered column order (qperm_pos): the dphiQ product below reads its rows in
        // accumulator-pair K order as single 16-byte reads
        for (int e2 = tid; e2 < K::C * D; e2 += K::NT) {
            const int i = e2 / D, col = e2 % D;
            sG[i * K::PV + qperm_pos(col)] = float_to_bf16_bits(bf16_bits_to_float(sDY[i * K::PV + col]) * sDn[i]);
            // d = 16: the group's other half is padding, which the staged y (read above) shares
            if (D < 32) sG[i * K::PV + qperm_pos(col + 16)] = 0;
        }
        __syncthreads();
        if (MODE == BW_CAUSAL) bwd_mtile<D, DP, MODE>(sG, sV, sC, sM, w, g, r16);
        __syncthreads();
        // ---- dphiQ for this wave's features: G S^T + c z^T (+ M phiK within the chunk, causal)
        bf16x8 sop[K::KSV][K::FBW];
#pragma unroll
        for (int ks = 0; ks < K::KSV; ks++)
#pragma unroll
            for (int j = 0; j < K::FBW; j++)
                sop[ks][j] = (2 * ks + 1 < K::VB) ? acc_pair_to_operand(ST[2 * ks][j], ST[2 * ks + 1][j])
                                                  : acc_pair_to_operand(ST[2 * ks][j], zero4());
#pragma unroll
        for (int ib = 0; ib < 4; ib++) {
#pragma unroll
            for (int j = 0; j < K::FBW; j++) {
                const int fb = K::FBW * w + j;
                f32x4 o = zero4();
                const bf16_t *grow = sG + (16 * ib + r16) * K::PV;
#pragma unroll
                for (int ks = 0; ks < K::KSV; ks++)
                    o = mfma_bf16(*reinterpret_cast<const bf16x8 *>(grow + 32 * ks + 8 * g), sop[ks][j], o);
                if (MODE == BW_CAUSAL) {
                    const bf16_t *mrow = sM + (16 * ib + r16) * K::PM;
#pragma unroll
                    for (int ks = 0; ks <= ib / 2; ks++)
                        o = mfma_bf16(*reinterpret_cast<const bf16x8 *>(mrow + 32 * ks + 8 * g),
                                      down_rows(sK, lr * K::PF + lo, 32 * ks, 16 * fb, K::PF), o);
                }
                // lane: feature 16 fb + r16, queries 16 ib + 4 g + r.  Each store takes a uniform row
                // base and the lane's 32-bit offset, so that no per-store 64-bit lane address stays
                // live across the chunk loop.
                // (c of the lane's four queries in one read, and validity as a count, for the same
                // reason: per-query addresses and indices would be kept live across the loop)
                const float zf = sZ[16 * fb + r16];
                const uint32_t lane_off = (uint32_t)(4 * g * DP + 16 * fb + r16);
                const f32x4 cq = *reinterpret_cast<const f32x4 *>(sC + 16 * ib + 4 * g);
                const int rem = valid - 16 * ib - 4 * g;
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    o[r] = fmaf(cq[r], zf, o[r]);
                    bf16_t *row = p.dphiq + (tok_base + t0 + 16 * ib + r) * DP;
                    if (r < rem && 16 * fb + r16 < DP) row[lane_off] = float_to_bf16_bits(o[r]);
                }
            }
        }
        // ---- this segment's reverse sums: R += phiQ^T G (by value columns), r += phiQ^T c (by features)
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
            // value columns 16 w .. 16 w + 15 of G down its rows: each lane addresses its 4-column
            // run where the reordering put it
            const bf16_t *gp = sG + (lr + 32 * ks) * K::PV + qperm_pos(16 * w + lo);
            const bf16x8 gop = cat(tr_read(gp), tr_read(gp + 4 * K::PV));
#pragma unroll
            for (int fb = 0; fb < K::FB; fb++)
                Racc[fb] = mfma_bf16(down_rows(sQ, lr * K::PF + lo, 32 * ks, 16 * fb, K::PF), gop, Racc[fb]);
            bf16x8 cop;
#pragma unroll
            for (int e2 = 0; e2 < 8; e2++) cop[e2] = (__bf16)sC[32 * ks + 8 * g + e2];
#pragma unroll
            for (int j = 0; j < K::FBW; j++)
                racc[j] = mfma_bf16(cop, down_rows(sQ, lr * K::PF + lo, 32 * ks, 16 * (K::FBW * w + j), K::PF), racc[j]);
        }
        // ---- forward sums with this chunk (causal): S^T += V^T phiK, z += phiK^T 1
        if (MODE == BW_CAUSAL) {
            f32x4 zacc[K::FBW];
#pragma unroll
            for (int j = 0; j < K::FBW; j++) zacc[j] = zero4();
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                bf16x8 kop[K::FBW];
#pragma unroll
                for (int j = 0; j < K::FBW; j++) kop[j] = down_rows(sK, lr * K::PF + lo, 32 * ks, 16 * (K::FBW * w + j), K::PF);
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++) {
                    const bf16x8 vop = down_rows(sV, lr * K::PV + lo, 32 * ks, 16 * vb, K::PV);
#pragma unroll
                    for (int j = 0; j < K::FBW; j++) ST[vb][j] = mfma_bf16(vop, kop[j], ST[vb][j]);
                }
#pragma unroll
                for (int j = 0; j < K::FBW; j++) zacc[j] = mfma_bf16(ones, kop[j], zacc[j]);
            }
            __syncthreads();  // every wave has read sZ for this chunk
            if (g == 0) {
#pragma unroll
                for (int j = 0; j < K::FBW; j++) sZ[16 * (K::FBW * w + j) + r16] += zacc[j][0];
            }
        }
        __syncthreads();
    }
    // ---- the segment's reverse-sum aggregate, canonical [DPP][D] then r [DPP]
    const long slot = MODE == BW_CAUSAL ? (s > 0 ? (long)bh * p.nseg + (p.nseg - 1 - s) : -1) : (long)bh * p.nseg + s;
    if (slot >= 0) {
        float *Rs = p.R_slots + slot * (long)K::DPP * D;
#pragma unroll
        for (int fb = 0; fb < K::FB; fb++)
#pragma unroll
            for (int r = 0; r < 4; r++) Rs[(size_t)(16 * fb + 4 * g + r) * D + 16 * w + r16] = Racc[fb][r];
        float *rs = p.r_slots + slot * (long)K::DPP;
        if (g == 0) {
#pragma unroll
            for (int j = 0; j < K::FBW; j++) rs[16 * (K::FBW * w + j) + r16] = racc[j][0];
        }
    }
}

// ---- k side ----------------------------------------------------------------------------
template <int D, int DP, int MODE>
__device__ void bwd_k_body(const BwdParams &p, unsigned char *smem, int bh, int s) {
    using K = BwdCfg<D, DP>;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int t_begin = s * p.seg_len, t_end = min(p.N, t_begin + p.seg_len);
    const int n = (t_end - t_begin + K::C - 1) / K::C;
    const size_t tok_base = (size_t)bh * p.N;
    bf16_t *sQ = reinterpret_cast<bf16_t *>(smem + K::OFF_Q), *sK = reinterpret_cast<bf16_t *>(smem + K::OFF_K);
    bf16_t *sV = reinterpret_cast<bf16_t *>(smem + K::OFF_V), *sG = reinterpret_cast<bf16_t *>(smem + K::OFF_G);
    bf16_t *sDY = reinterpret_cast<bf16_t *>(smem + K::OFF_DY);
    bf16_t *sM = reinterpret_cast<bf16_t *>(smem + K::OFF_M), *sP = reinterpret_cast<bf16_t *>(smem + K::OFF_P);
    float *sRS = reinterpret_cast<float *>(smem + K::OFF_F32) + K::NW * K::C;
    float *sDn = sRS + 4 * K::C, *sC = sDn + K::C;
    float *sR = sC + K::C;  // r per feature (after the chunk)

    for (int i = tid; i < K::LDS_BYTES / 16; i += K::NT) reinterpret_cast<f32x4 *>(smem)[i] = zero4();
    __syncthreads();

    // R^T by features: RT[vb][j] rows value columns 16 vb + 4 g + r, column feature 16 (FBW w + j) + r16;
    // R by value columns: RV[fb] rows features 16 fb + 4 g + r, column value 16 w + r16
    f32x4 RT[K::VB][K::FBW], RV[K::FB], racc[K::FBW];
#pragma unroll
    for (int vb = 0; vb < K::VB; vb++)
#pragma unroll
        for (int j = 0; j < K::FBW; j++) RT[vb][j] = zero4();
#pragma unroll
    for (int fb = 0; fb < K::FB; fb++) RV[fb] = zero4();
#pragma unroll
    for (int j = 0; j < K::FBW; j++) racc[j] = zero4();
    {
        // sums over the later segments (causal: slot nseg-1-s holds their exclusive prefix in
        // reversed order; the last segment has none) or over all (bidirectional: slot 0)
        const long sl = MODE == BW_CAUSAL ? (s < p.nseg - 1 ? (long)bh * p.nseg + (p.nseg - 1 - s) : -1)
                                          : (long)bh * p.nseg;
        if (sl >= 0) {
            const float *Rp = p.R_slots + sl * (long)K::DPP * D;
            const float *rp = p.r_slots + sl * (long)K::DPP;
#pragma unroll
            for (int vb = 0; vb < K::VB; vb++)
#pragma unroll
                for (int j = 0; j < K::FBW; j++)
                    RT[vb][j] = *reinterpret_cast<const f32x4 *>(Rp + (size_t)(16 * (K::FBW * w + j) + r16) * D + 16 * vb + 4 * g);
#pragma unroll
            for (int fb = 0; fb < K::FB; fb++)
#pragma unroll
                for (int r = 0; r < 4; r++) RV[fb][r] = Rp[(size_t)(16 * fb + 4 * g + r) * D + 16 * w + r16];
            for (int f = tid; f < K::DPP; f += K::NT) sR[f] = rp[f];
        }
    }
    __syncthreads();

    const int lo = 4 * (r16 & 3);
    const int lr = 8 * g + (r16 >> 2);
    for (int c = n - 1; c >= 0; c--) {
        const int t0 = t_begin + K::C * c;
        const int valid = min(K::C, t_end - t0);
        // den and c of the chunk's queries, requested with the staging loads (one memory wait)
        float2 dc = make_float2(1.0f, 0.0f);
        const bool dc_live = tid < K::C && tid < valid;
        if (dc_live) dc = *reinterpret_cast<const float2 *>(p.den_c + 2 * (tok_base + t0 + tid));
        bwd_stage<D, DP, false, true>(p, tok_base + t0, valid, smem, tid);
        if (tid < K::C) {
            sDn[tid] = dc_live ? 1.0f / dc.x : 0.0f;
            sC[tid] = dc_live ? dc.y : 0.0f;
        }
        __syncthreads();
        for (int e2 = tid; e2 < K::C * D; e2 += K::NT) {
            const int i = e2 / D, col = e2 % D;
            sG[i * K::PV + col] = float_to_bf16_bits(bf16_bits_to_float(sDY[i * K::PV + col]) * sDn[i]);
        }
        if (MODE == BW_CAUSAL) bwd_scores_t<D, DP, MODE>(sQ, sK, sP, w, g, r16);
        __syncthreads();
        if (MODE == BW_CAUSAL) bwd_mtile_t<D, DP, MODE>(sG, sV, sC, sM, w, g, r16);
        __syncthreads();
        // ---- dphiK for this wave's features: V R^T + r (+ M^T phiQ within the chunk, causal)
        bf16x8 rop[K::KSV][K::FBW];
#pragma unroll
        for (int ks = 0; ks < K::KSV; ks++)
#pragma unroll
            for (int j = 0; j < K::FBW; j++)
                rop[ks][j] = (2 * ks + 1 < K::VB) ? acc_pair_to_operand(RT[2 * ks][j], RT[2 * ks + 1][j])
                                                  : acc_pair_to_operand(RT[2 * ks][j], zero4());
#pragma unroll
        for (int jb = 0; jb < 4; jb++) {
#pragma unroll
            for (int j = 0; j < K::FBW; j++) {
                const int fb = K::FBW * w + j;
                f32x4 o = zero4();
                const bf16_t *vrow = sV + (16 * jb + r16) * K::PV;
#pragma unroll
                for (int ks = 0; ks < K::KSV; ks++)
                    o = mfma_bf16(*reinterpret_cast<const bf16x8 *>(vrow + 32 * ks + 8 * g), rop[ks][j], o);
                // M^T phiQ: A = M^T (row key, K queries), B = phiQ (K queries, column feature)
                if (MODE == BW_CAUSAL) {
#pragma unroll
                    for (int ks = 0; ks < 2; ks++) {
                        if (ks < jb / 2) continue;
                        o = mfma_bf16(*reinterpret_cast<const bf16x8 *>(sM + (16 * jb + r16) * K::PM + 32 * ks + 8 * g),
                                      down_rows(sQ, lr * K::PF + lo, 32 * ks, 16 * fb, K::PF), o);
                    }
                }
                const float rf = sR[16 * fb + r16];
                const uint32_t lane_off = (uint32_t)(4 * g * DP + 16 * fb + r16);
                const int rem = valid - 16 * jb - 4 * g;
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    bf16_t *row = p.dphik + (tok_base + t0 + 16 * jb + r) * DP;  // uniform row base
                    if (r < rem && 16 * fb + r16 < DP) row[lane_off] = float_to_bf16_bits(o[r] + rf);
                }
            }
        }
        // ---- dV for value block w (transposed: rows value columns, column key): R^T phiK^T + G^T P
        {
            bf16x8 rvop[K::KSF];
#pragma unroll
            for (int ks = 0; ks < K::KSF; ks++) rvop[ks] = acc_pair_to_operand(RV[2 * ks], RV[2 * ks + 1]);
#pragma unroll
            for (int jb = 0; jb < 4; jb++) {
                f32x4 o = zero4();
                const bf16_t *krow = sK + (16 * jb + r16) * K::PF;
#pragma unroll
                for (int ks = 0; ks < K::KSF; ks++)
                    o = mfma_bf16(rvop[ks], *reinterpret_cast<const bf16x8 *>(krow + 32 * ks + 8 * g), o);
                if (MODE == BW_CAUSAL) {
#pragma unroll
                    for (int ks = 0; ks < 2; ks++) {
                        if (ks < jb / 2) continue;
                        o = mfma_bf16(down_rows(sG, lr * K::PV + lo, 32 * ks, 16 * w, K::PV),
                                      *reinterpret_cast<const bf16x8 *>(sP + (16 * jb + r16) * K::PM + 32 * ks + 8 * g), o);
                    }
                }
                const int jj = 16 * jb + r16;
                if (jj < valid) {
                    bf16_t *dst = p.dv + (tok_base + t0 + jj) * D + 16 * w + 4 * g;
                    store4(dst, to_bf16x4(o));
                }
            }
        }
        // ---- reverse sums with this chunk (causal): R^T += G^T phiQ, R += phiQ^T G, r += phiQ^T c
        if (MODE == BW_CAUSAL) {
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                bf16x8 qop[K::FBW];
#pragma unroll
                for (int j = 0; j < K::FBW; j++) qop[j] = down_rows(sQ, lr * K::PF + lo, 32 * ks, 16 * (K::FBW * w + j), K::PF);
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++) {
                    const bf16x8 gop = down_rows(sG, lr * K::PV + lo, 32 * ks, 16 * vb, K::PV);
#pragma unroll
                    for (int j = 0; j < K::FBW; j++) RT[vb][j] = mfma_bf16(gop, qop[j], RT[vb][j]);
                }
                const bf16x8 gw = down_rows(sG, lr * K::PV + lo, 32 * ks, 16 * w, K::PV);
#pragma unroll
                for (int fb = 0; fb < K::FB; fb++)
                    RV[fb] = mfma_bf16(down_rows(sQ, lr * K::PF + lo, 32 * ks, 16 * fb, K::PF), gw, RV[fb]);
                bf16x8 cop;
#pragma unroll
                for (int e2 = 0; e2 < 8; e2++) cop[e2] = (__bf16)sC[32 * ks + 8 * g + e2];
#pragma unroll
                for (int j = 0; j < K::FBW; j++) racc[j] = mfma_bf16(cop, qop[j], racc[j]);
            }
        }
        __syncthreads();  // every wave has read sR and the tiles
        if (MODE == BW_CAUSAL && g == 0) {
#pragma unroll
            for (int j = 0; j < K::FBW; j++) sR[16 * (K::FBW * w + j) + r16] += racc[j][0];
        }
#pragma unroll
        for (int j = 0; j < K::FBW; j++) racc[j] = zero4();
        __syncthreads();
    }
}

template <int D, int DP, int MODE>
__global__ __launch_bounds__(4 * D) void bwd_q_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[BwdCfg<D, DP>::LDS_BYTES];
    int bh, s;
    head_segment(p.nseg, bh, s);
    bwd_q_body<D, DP, MODE>(p, smem, bh, s);
}

template <int D, int DP, int MODE>
__global__ __launch_bounds__(4 * D) void bwd_k_kernel(BwdParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[BwdCfg<D, DP>::LDS_BYTES];
    int bh, s;
    head_segment(p.nseg, bh, s);
    bwd_k_body<D, DP, MODE>(p, smem, bh, s);
}

// ---- feature-map backward ----------------------------------------------------------------
// One workgroup (4 waves) per TILES64 x 64 tokens of one sequence, for q and for k: u^T = W x^T
// recomputed (lane: token r16, directions 16 lb + 4 g + r), dL/du from dL/dphi by the map's
// chain rule, dx = W^T du on the matrix cores, and this workgroup's part of dW = sum du x^T and
// db = sum du (du and x through LDS as [token][.] tiles, read transposed).
constexpr int kMapTiles = 4;  // 64-token tiles per workgroup (per input)

template <int D>
struct MapCfg {
    static constexpr int LB = D / 16, KS = (D + 31) / 32, DK = KS * 32;
    static constexpr int PX = pitch_of(DK), PW = pitch_of(D);
    static constexpr int OFF_W = 0;                        // W [l][m], pitch PW, DK rows (rows >= D zero)
    static constexpr int OFF_X = OFF_W + DK * PW * 2;      // x tile [64][PX]
    static constexpr int OFF_U = OFF_X + 64 * PX * 2;      // du tile [64][PX] (bf16)
    static constexpr int OFF_B = OFF_U + 64 * PX * 2;      // bias [D] (fp32)
    static constexpr int LDS_BYTES = OFF_B + D * 4;
    static constexpr int NX = 64 * D / 8;                  // 16-byte pieces of an x tile
    static constexpr int PERX = (NX + 255) / 256;          // per thread
};

// At least two waves per SIMD (two workgroups per CU, as the LDS allows): left free, the
// compiler takes more than 256 registers (VGPRs plus AGPRs used as spill space) and runs one.
// The two-sided softmax map's backward would spill at that budget and keeps one.
template <int D, int MAP>
__global__ __launch_bounds__(256, MAP == HH_MAP_HEDGEHOG_SOFTMAX_ ? 1 : 2) void bwd_map_kernel(BwdParams p, int tiles_per_seq,
                                                                                                int wgs_per_seq) {
    using K = MapCfg<D>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[K::LDS_BYTES];
    constexpr bool TWO = MAP == HH_MAP_HEDGEHOG_ || MAP == HH_MAP_HEDGEHOG_SOFTMAX_;  // two-sided maps
    constexpr int DP = TWO ? 2 * D : D;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const long bh = blockIdx.x / wgs_per_seq;
    const int part = blockIdx.x % wgs_per_seq;
    const int h = (int)(bh % p.H);
    const bf16_t *Wh = p.W + (size_t)h * D * D;
    bf16_t *sW = reinterpret_cast<bf16_t *>(smem + K::OFF_W);
    bf16_t *sX = reinterpret_cast<bf16_t *>(smem + K::OFF_X);
    bf16_t *sU = reinterpret_cast<bf16_t *>(smem + K::OFF_U);
    float *sB = reinterpret_cast<float *>(smem + K::OFF_B);
    for (int i = tid; i < K::OFF_B / 16; i += 256) reinterpret_cast<f32x4 *>(smem)[i] = zero4();
    if (tid < D) sB[tid] = p.b ? bf16_bits_to_float(p.b[(size_t)h * D + tid]) : 0.0f;
    __syncthreads();
    stage_pieces<256, D * D / 8>(
        tid, [&](int e) { return Wh + 8 * e; }, [&](int e) { return sW + (e / (D / 8)) * K::PW + 8 * (e % (D / 8)); },
        [](int) { return true; });
    // dW part: blocks (lb, mb) dealt over the 4 waves; db part: the ones trick
    constexpr int NBLK = (D / 16) * (D / 16);
    constexpr int BPW = (NBLK + 3) / 4;
    constexpr int NMB = K::LB >= 8 ? 2 : 1;  // input-dim blocks of a wave's dW blocks: mb = (wv + 4 i) % LB
    f32x4 dWacc[BPW];
#pragma unroll
    for (int i = 0; i < BPW; i++) dWacc[i] = zero4();
    f32x4 dbacc[2] = {zero4(), zero4()};  // direction blocks wv and wv + 4
    const bf16x8 ones = ones_bf16x8();
    const int lr = 8 * g + (r16 >> 2), lo = 4 * (r16 & 3);
    const int lrp = 4 * g + (r16 >> 2);

    // Tiles of this workgroup: the same ntl tiles of q, then of k.  Tile j's x and dL/dphi are
    // requested as soon as tile j - 1 has formed du, so that they arrive during its dx and dW
    // products (requested any earlier, the wait for tile j - 1's dL/dphi would also wait for
    // them: loads retire in order).  Rows past the end are loaded from a stand-in row and zeroed
    // when stored (a select right after a load would wait for it).
    const int ntl = min(kMapTiles, tiles_per_seq - part * kMapTiles);
    const int nit = 2 * ntl;
    bf16x8 xbuf[K::PERX];
    auto x_src = [&](int j) { return j < ntl ? p.q : p.k; };
    auto n0_of = [&](int j) { return (part * kMapTiles + (j < ntl ? j : j - ntl)) * 64; };
    auto load_x = [&](int j) {
        const bf16_t *x = x_src(j);
        const int n0 = n0_of(j);
#pragma unroll
        for (int i = 0; i < K::PERX; i++) {
            const int e = tid + 256 * i;
            const bool ok = (K::NX % 256 == 0 || e < K::NX) && n0 + e / (D / 8) < p.N;
            const int row = ok ? n0 + e / (D / 8) : 0;  // a stand-in row where there is none
            xbuf[i] = load8(x + ((size_t)bh * p.N + row) * D + 8 * (e % (D / 8)));
        }
    };
    auto store_x = [&](int j) {
        const int n0 = n0_of(j);
#pragma unroll
        for (int i = 0; i < K::PERX; i++) {
            const int e = tid + 256 * i;
            if (K::NX % 256 == 0 || e < K::NX)
                store8(sX + (e / (D / 8)) * K::PX + 8 * (e % (D / 8)), n0 + e / (D / 8) < p.N ? xbuf[i] : zero_bf16x8());
        }
    };
    // dL/dphi of the lane's token (its directions, and for two-sided maps their negations)
    auto load_dphi = [&](int j, bf16x4 (&da)[K::LB], bf16x4 (&db_)[K::LB]) {
        const int nn = n0_of(j) + 16 * wv + r16;
        const size_t tok = (size_t)bh * p.N + (nn < p.N ? nn : 0);
        const bf16_t *dp_ = (j < ntl ? p.dphiq : p.dphik) + tok * DP;
#pragma unroll
        for (int lb = 0; lb < K::LB; lb++) {
            da[lb] = load4(dp_ + 16 * lb + 4 * g);
            db_[lb] = TWO ? load4(dp_ + D + 16 * lb + 4 * g) : to_bf16x4(zero4());
        }
    };

    bf16x4 dpa16[K::LB], dpb16[K::LB];
    auto tile = [&](int j) {
        store_x(j);
        __syncthreads();
        const int n0 = n0_of(j);
        const int nn = n0 + 16 * wv + r16;  // this lane's token
        const bool live = nn < p.N;
        const size_t tok = (size_t)bh * p.N + (live ? nn : 0);
        bf16_t *dx = j < ntl ? p.dq : p.dk;
        // u^T: A = W rows (directions), B = x^T (token r16)
        f32x4 u[K::LB];
#pragma unroll
        for (int lb = 0; lb < K::LB; lb++) {
            u[lb] = *reinterpret_cast<const f32x4 *>(sB + 16 * lb + 4 * g);  // the bias
#pragma unroll
            for (int ks = 0; ks < K::KS; ks++) {
                const bf16x8 wa = (32 * ks + 8 * g < D) ? *reinterpret_cast<const bf16x8 *>(sW + (16 * lb + r16) * K::PW + 32 * ks + 8 * g)
                                                        : zero_bf16x8();
                u[lb] = mfma_bf16(wa, *reinterpret_cast<const bf16x8 *>(sX + (16 * wv + r16) * K::PX + 32 * ks + 8 * g), u[lb]);
            }
        }
        // dL/du for directions 16 lb + 4 g + r of token r16
        f32x4 du[K::LB];
        if (MAP == HH_MAP_HEDGEHOG_ || MAP == HH_MAP_EXP_) {
#pragma unroll
            for (int lb = 0; lb < K::LB; lb++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const float uu = u[lb][r];
                    float v = (float)dpa16[lb][r] * __expf(uu);
                    if (MAP == HH_MAP_HEDGEHOG_) v -= (float)dpb16[lb][r] * __expf(-uu);
                    du[lb][r] = v;
                }
        } else {
#pragma unroll
            for (int lb = 0; lb < K::LB; lb++) du[lb] = zero4();
#pragma unroll
            for (int half = 0; half < (MAP == HH_MAP_HEDGEHOG_SOFTMAX_ ? 2 : 1); half++) {
                const float sg = half ? -1.0f : 1.0f;
                float mx = -INFINITY;
#pragma unroll
                for (int lb = 0; lb < K::LB; lb++)
#pragma unroll
                    for (int r = 0; r < 4; r++) mx = fmaxf(mx, sg * u[lb][r]);
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                f32x4 e[K::LB], dpv[K::LB];
                float sum = 0.0f, dot = 0.0f;
#pragma unroll
                for (int lb = 0; lb < K::LB; lb++) {
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        dpv[lb][r] = (float)(half ? dpb16[lb][r] : dpa16[lb][r]);
                        e[lb][r] = __expf(sg * u[lb][r] - mx);
                        sum += e[lb][r];
                    }
                }
                sum += __shfl_xor(sum, 16);
                sum += __shfl_xor(sum, 32);
                const float rs = 1.0f / sum;
#pragma unroll
                for (int lb = 0; lb < K::LB; lb++)
#pragma unroll
                    for (int r = 0; r < 4; r++) dot = fmaf(dpv[lb][r], e[lb][r] * rs, dot);
                dot += __shfl_xor(dot, 16);
                dot += __shfl_xor(dot, 32);
#pragma unroll
                for (int lb = 0; lb < K::LB; lb++)
#pragma unroll
                    for (int r = 0; r < 4; r++) du[lb][r] += sg * e[lb][r] * rs * (dpv[lb][r] - dot);
            }
        }
        if (!live) {
#pragma unroll
            for (int lb = 0; lb < K::LB; lb++) du[lb] = zero4();
        }
        if (j + 1 < nit) {
            load_x(j + 1);
            load_dphi(j + 1, dpa16, dpb16);
        }
        // du tile [token][direction] (bf16) for the dW part
#pragma unroll
        for (int lb = 0; lb < K::LB; lb++) store4(sU + (16 * wv + r16) * K::PX + 16 * lb + 4 * g, to_bf16x4(du[lb]));
        // dx^T = W^T du: rows input dims, column token; A = W^T (rows m, K directions in the
        // accumulator pair order), B = du pair
#pragma unroll
        for (int mb = 0; mb < D / 16; mb++) {
            f32x4 o = zero4();
#pragma unroll
            for (int ks = 0; ks < K::KS; ks++) {
                const bf16x8 bop = (2 * ks + 1 < K::LB) ? acc_pair_to_operand(du[2 * ks], du[2 * ks + 1])
                                                        : acc_pair_to_operand(du[2 * ks], zero4());
                o = mfma_bf16(down_rows_perm(sW, lrp * K::PW + lo, 32 * ks, 16 * mb, K::PW), bop, o);
            }
            if (live) store4(dx + tok * D + 16 * mb + 4 * g, to_bf16x4(o));
        }
        __syncthreads();
        // dW part += du^T x over the tile's tokens: A = du^T (rows directions, K tokens),
        // B = x (K tokens, column input dim); db part += du^T 1.  Each operand read once.
        bf16x8 xop[NMB][2];
#pragma unroll
        for (int m = 0; m < NMB; m++)
#pragma unroll
            for (int ks = 0; ks < 2; ks++) xop[m][ks] = down_rows(sX, lr * K::PX + lo, 32 * ks, 16 * ((wv + 4 * m) % K::LB), K::PX);
        bf16x8 uop[2];
#pragma unroll
        for (int i = 0; i < BPW; i++) {
            const int blk = wv + 4 * i;
            if (blk >= NBLK) continue;
            const int lb = blk / K::LB;
            if (i % NMB == 0) {
#pragma unroll
                for (int ks = 0; ks < 2; ks++) uop[ks] = down_rows(sU, lr * K::PX + lo, 32 * ks, 16 * lb, K::PX);
            }
#pragma unroll
            for (int ks = 0; ks < 2; ks++) dWacc[i] = mfma_bf16(uop[ks], xop[i % NMB][ks], dWacc[i]);
        }
#pragma unroll
        for (int hb = 0; hb < 2; hb++) {
            const int lb = wv + 4 * hb;
            if (lb >= K::LB) continue;
#pragma unroll
            for (int ks = 0; ks < 2; ks++)
                dbacc[hb] = mfma_bf16(down_rows(sU, lr * K::PX + lo, 32 * ks, 16 * lb, K::PX), ones, dbacc[hb]);
        }
        __syncthreads();
    };

    if (nit > 0) {
        load_x(0);
        load_dphi(0, dpa16, dpb16);
    }
    __syncthreads();  // W staged
    for (int j = 0; j < nit; j++) tile(j);
    // this workgroup's parts: dW [D][D] rows directions 16 lb + 4 g + r, column input dim 16 mb + r16
    float *dWp = p.dW_parts + (size_t)blockIdx.x * (D * D + D);
#pragma unroll
    for (int i = 0; i < BPW; i++) {
        const int blk = wv + 4 * i;
        if (blk >= NBLK) continue;
        const int lb = blk / (D / 16), mb = blk % (D / 16);
#pragma unroll
        for (int r = 0; r < 4; r++) dWp[(size_t)(16 * lb + 4 * g + r) * D + 16 * mb + r16] = dWacc[i][r];
    }
    // db: direction blocks wv and wv + 4
    if (r16 == 0) {
#pragma unroll
        for (int hb = 0; hb < 2; hb++) {
            const int lb = wv + 4 * hb;
            if (lb >= K::LB) continue;
#pragma unroll
            for (int r = 0; r < 4; r++) dWp[D * D + 16 * lb + 4 * g + r] = dbacc[hb][r];
        }
    }
}

// dW[h] = sum over (b, workgroup) of the parts; db likewise.  One thread per entry.
__global__ void bwd_reduce_kernel(const float *__restrict__ parts, float *__restrict__ dW, float *__restrict__ db, int B,
                                  int H, int d, int wgs_per_seq) {
    const long per = (long)d * d + d;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)H * per) return;
    const int h = (int)(idx / per);
    const long e = idx % per;
    // parts in groups of 16 with every load of a group issued before its sums (a load-then-add
    // loop would wait one memory latency per part); the sum order is the parts' order
    float acc = 0.0f;
    for (int b = 0; b < B; b++) {
        const float *pb = parts + (size_t)(b * H + h) * wgs_per_seq * per + e;
        for (int w0 = 0; w0 < wgs_per_seq; w0 += 16) {
            float v[16];
#pragma unroll
            for (int j = 0; j < 16; j++) {
                const int wg = w0 + j < wgs_per_seq ? w0 + j : w0;  // a stand-in part past the end, not added
                v[j] = pb[(size_t)wg * per];
            }
            __builtin_amdgcn_sched_barrier(0);  // the group's loads all in flight before the first sum
#pragma unroll
            for (int j = 0; j < 16; j++) acc += w0 + j < wgs_per_seq ? v[j] : 0.0f;
        }
    }
    if (e < (long)d * d) dW[(size_t)h * d * d + e] = acc;
    else if (db) db[(size_t)h * d + (e - (long)d * d)] = acc;
}

template <int D, int DP>
hipError_t launch_bwd_d(int which, int causal, const BwdParams &p, int grid, hipStream_t st) {
    if (which == 0) {
        if (causal) hipLaunchKernelGGL((bwd_q_kernel<D, DP, BW_CAUSAL>), dim3(grid), dim3(4 * D), 0, st, p);
        else hipLaunchKernelGGL((bwd_q_kernel<D, DP, BW_BIDIR>), dim3(grid), dim3(4 * D), 0, st, p);
    } else {
        if (causal) hipLaunchKernelGGL((bwd_k_kernel<D, DP, BW_CAUSAL>), dim3(grid), dim3(4 * D), 0, st, p);
        else hipLaunchKernelGGL((bwd_k_kernel<D, DP, BW_BIDIR>), dim3(grid), dim3(4 * D), 0, st, p);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_map_d(int map, const BwdParams &p, int tiles, int wgs, int grid, hipStream_t st) {
    switch (map) {
    case HH_MAP_HEDGEHOG_: hipLaunchKernelGGL((bwd_map_kernel<D, HH_MAP_HEDGEHOG_>), dim3(grid), dim3(256), 0, st, p, tiles, wgs); break;
    case HH_MAP_EXP_: hipLaunchKernelGGL((bwd_map_kernel<D, HH_MAP_EXP_>), dim3(grid), dim3(256), 0, st, p, tiles, wgs); break;
    case HH_MAP_SOFTMAX_: hipLaunchKernelGGL((bwd_map_kernel<D, HH_MAP_SOFTMAX_>), dim3(grid), dim3(256), 0, st, p, tiles, wgs); break;
    default: hipLaunchKernelGGL((bwd_map_kernel<D, HH_MAP_HEDGEHOG_SOFTMAX_>), dim3(grid), dim3(256), 0, st, p, tiles, wgs); break;
    }
    return hipGetLastError();
}

}  // namespace

int bwd_wgs_per_seq(int N) { return ((N + 63) / 64 + kMapTiles - 1) / kMapTiles; }

hipError_t launch_bwd_pass(int which, int d, int dp, int causal, const BwdParams &p, int grid, hipStream_t st) {
    switch (d * 1000 + dp) {
    case 16016: return launch_bwd_d<16, 16>(which, causal, p, grid, st);
    case 16032: return launch_bwd_d<16, 32>(which, causal, p, grid, st);
    case 32032: return launch_bwd_d<32, 32>(which, causal, p, grid, st);
    case 32064: return launch_bwd_d<32, 64>(which, causal, p, grid, st);
    case 64064: return launch_bwd_d<64, 64>(which, causal, p, grid, st);
    case 64128: return launch_bwd_d<64, 128>(which, causal, p, grid, st);
    case 128128: return launch_bwd_d<128, 128>(which, causal, p, grid, st);
    case 128256: return launch_bwd_d<128, 256>(which, causal, p, grid, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd_map(int map, int d, const BwdParams &p, long BH, hipStream_t st) {
    const int tiles = (p.N + 63) / 64, wgs = bwd_wgs_per_seq(p.N);
    const int grid = (int)(BH * wgs);
    switch (d) {
    case 16: return launch_map_d<16>(map, p, tiles, wgs, grid, st);
    case 32: return launch_map_d<32>(map, p, tiles, wgs, grid, st);
    case 64: return launch_map_d<64>(map, p, tiles, wgs, grid, st);
    case 128: return launch_map_d<128>(map, p, tiles, wgs, grid, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd_reduce(const float *parts, float *dW, float *db, int B, int H, int d, int N, hipStream_t st) {
    const long total = (long)H * ((long)d * d + d);
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, parts, dW, db, B, H, d,
                       bwd_wgs_per_seq(N));
    return hipGetLastError();
}

}  // namespace hh
