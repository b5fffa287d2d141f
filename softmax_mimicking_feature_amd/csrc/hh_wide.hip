// hh_wide.hip -- chunked Hedgehog linear attention on the CDNA4 matrix cores (bf16 in, fp32 state).
//
// What is computed (paper-graph-ui walkthrough of "The Hedgehog & the
// Porcupine", section 2 Eq. 2 and section 3.4 "Complexity Analysis"):
//     y_i = phi(q_i)^T S_i / phi(q_i)^T z_i,   S_i = sum_{j<=i} phi(k_j) v_j^T,  z_i = sum_{j<=i} phi(k_j)
// with phi(x) = [exp(W x + b), exp(-(W x + b))] (section 3.4, Choices 1 and 3).
//
// How: the sequence of one (batch, head) is cut into segments, each segment
// into chunks of C = 64 tokens.  Per chunk, with Sp, zp the state before it:
//     y_c = (phiQ_c Sp + tril(phiQ_c phiK_c^T) V_c) / (phiQ_c zp + tril(phiQ_c phiK_c^T) 1)
//     Sp += phiK_c^T V_c,  zp += phiK_c^T 1
// which regroups the running sums of Eq. 2 exactly (only rounding differs).
// Three modes of one kernel template:
//   STATE   : segment aggregate dS = phiK^T V, dz = phiK^T 1 over the segment -> workspace
//   CAUSAL  : the chunk recurrence above, starting from the segment's prefix state
//   READOUT : y = phiQ S / phiQ z against a fixed total state (bidirectional mode)
// A separate scan kernel turns segment aggregates into exclusive prefixes.
//
// Work split inside a workgroup of NW waves (one wave per SIMD):
//   feature map : wave w computes directions [16 LB w, 16 LB (w+1)) for all 64 tokens
//                 (u^T = W x^T on MFMA, W rows held in registers), exp epilogue -> LDS
//   scores      : wave w computes query blocks [IBW w, IBW (w+1)) against key blocks <= them
//   read-out, intra-chunk product, state update: wave w owns value columns
//                 [16 VB w, 16 VB (w+1)) of S for every feature row, kept as fp32
//                 accumulators in registers for the whole segment
//   normaliser z: rows of z are split across waves; partial denominators meet in LDS.
#include "hh_common.h"
#include "hh_kernels.h"

namespace hh {

// Row stride (elements) of a bf16 tile read with the transposing LDS load: rows start
// 32 bytes apart modulo 128 bytes, so the four rows one 16-lane group reads fall in
// disjoint banks.
constexpr int tr_stride(int n) { return n + ((((32 - 2 * n) % 128) + 128) % 128) / 2; }

enum { WM_STATE = 0, WM_CAUSAL = 1, WM_READOUT = 2 };

template <int D, int C_ = 64, int MODE_ = WM_CAUSAL>
struct WideCfg {
    static constexpr int C = C_;                      // tokens per chunk
    static constexpr int MODE = MODE_;
    static constexpr int NCB = C / 16;                // 16-token blocks per chunk
    static constexpr int KSC = C / 32;                // 32-wide K steps over the chunk's tokens
    static constexpr int NW = D == 128 ? 8 : (D == 64 ? 4 : D / 16);  // waves per workgroup
    static constexpr int NT = NW * 64;
    static constexpr int DP = 2 * D;                  // feature dimension
    static constexpr int FB = DP / 16;                // 16-row feature blocks
    static constexpr int KSF = DP / 32;               // 32-wide K steps over features
    static constexpr int KSD = (D + 31) / 32;         // K steps over the head dim (D = 16: half-filled)
    // feature map: NTH token groups x NDQ direction groups
    static constexpr int NTH = NW == 8 ? 2 : 1;
    static constexpr int NDQ = NW / NTH;
    static constexpr int DPW = D / NDQ;               // directions per wave
    static constexpr int LB = DPW / 16;               // direction blocks per wave
    static constexpr int IBT = NCB / NTH;             // token blocks per wave in the feature map
    // state: NF feature parts x NN value-column parts
    static constexpr int NF = NW == 8 ? 2 : 1;
    static constexpr int NN = NW / NF;
    static constexpr int VB = D / 16 / NN;            // value-column blocks per wave
    static constexpr int FBW = FB / NF;               // feature blocks per wave
    static constexpr int KSW = FBW / 2;               // read-out K steps per wave
    static constexpr int ZB = FB / NW;                // z-row blocks per wave
    static constexpr int IBF = NCB / NF;              // output row blocks finalised per wave
    static constexpr int IMG8 = FBW * VB / 2;         // accumulator pairs of a segment slot per lane
    static constexpr int NJ = (NW == 8) ? 2 : 1;      // intra-chunk row-sum slots
    // Staging buffers for the raw inputs.  With two (one workgroup per CU), q, k and V of the
    // next chunk are fetched straight into LDS a whole chunk ahead; with one (two workgroups
    // per CU), q and k are fetched after the feature maps have consumed the buffer and V goes
    // through registers.
    static constexpr int NBUF = D == 128 ? 2 : 1;
    static constexpr bool USE_Q = MODE != WM_STATE;
    static constexpr bool USE_K = MODE != WM_READOUT;
    static constexpr int VPT = NBUF == 1 ? C * (D / 8) / NT : 1;  // 16-byte pieces of V per thread and chunk
    // LDS tiles
    // Row strides of the feature tiles, chosen for the LDS bank mapping of gfx950 (measured):
    // 16-byte reads of 16 rows x 4 column blocks are conflict-free when the row pitch is 32
    // (mod 256) bytes; 8-byte writes of that shape and transposing reads with 16-byte-spaced
    // runs are conflict-free when it is an odd multiple of 8 bytes (mod 256).
    static constexpr int RQ = DP + 16;                // phi(q) [C][RQ]: 16-byte row reads and writes
    static constexpr int RK = DP + 12;                // phi(k) [C][RK]: 8-byte row reads, transposing reads
    // V [C][RV]: transposing reads.  Two buffers: unpadded 256-byte rows filled by direct loads,
    // 16-byte granules rotated by 4 per row (v_pos); one buffer: padded rows.
    static constexpr int RV = NBUF == 2 ? D : tr_stride(D);
    static constexpr int RA = C + 8;                  // intra scores A [C][RA]
    static constexpr int XS = D + 4;                  // fp32 exchange tile [C][XS] (NF = 2), aliases phi(q)
    // raw q / k of a chunk, loaded straight from global memory into LDS: [C][D] bf16, 16-byte
    // granules placed by stage_pos
    static constexpr int NG = D / 8;                  // 16-byte granules per row
    static constexpr int NSW = NG < 8 ? NG : 8;       // XOR swizzle period (rows of fewer than 16 granules)
    static constexpr int SZ_X = C * D * 2;
    static constexpr int XBLK = SZ_X / 1024;          // 1 KB direct-load blocks per tile
    static constexpr int SZ_PQ = !USE_Q ? 0 : ((C * RQ * 2 > (NF == 2 ? C * XS * 4 : 0)) ? C * RQ * 2 : C * XS * 4);
    static constexpr int SZ_PK = USE_K ? C * RK * 2 : 0;
    static constexpr int SZ_V1 = C * RV * 2;
    static constexpr int OFF_PQ = 0;
    static constexpr int OFF_PK = OFF_PQ + SZ_PQ;
    static constexpr int OFF_V = OFF_PK + SZ_PK;
    static constexpr int OFF_A = OFF_V + (USE_K ? NBUF * SZ_V1 : 0);
    static constexpr int OFF_DEN = OFF_A + (MODE == WM_CAUSAL ? C * RA * 2 : 0);
    static constexpr int OFF_XQ = OFF_DEN + (USE_Q ? (NW + NJ) * C * 4 : 0);
    static constexpr int OFF_XK = OFF_XQ + (USE_Q ? NBUF * SZ_X : 0);
    // per-head W, [D rows][D] bf16 with granule swizzle like the x tiles: only read once into
    // registers before the first chunk, so it shares the feature tiles' space
    static constexpr int OFF_W = OFF_PQ;
    static constexpr int LDS_BYTES = OFF_XK + (USE_K ? NBUF * SZ_X : 0);
    static constexpr int MIN_WG_PER_CU = NW == 8 ? 1 : 2;
    static_assert(ZB == 2, "each wave owns one K step of z rows");
    static_assert(VB >= 1 && LB >= 1 && IBT >= 1 && IBF >= 1 && FBW % 2 == 0, "bad wave split");
    static_assert(NBUF == 2 || (VPT >= 1 && C * (D / 8) % NT == 0), "every lane moves whole V pieces");
    static_assert(D * D * 2 <= SZ_PQ + SZ_PK, "W fits in the feature tiles");
    static_assert(SZ_X % 1024 == 0 && XBLK % NW == 0, "direct loads: whole 1 KB blocks, the same count per wave");
    static_assert(NBUF == 1 || (D == 128 && VB == 2), "rotated V tile assumes 16 granules per row");
};

// Segment slots keep S in fp32 in the register image of the kernel that reads them back:
// the two accumulators (halves h = 0, 1) that lane L of a wave holds as piece e are stored as
// f32x4 at index (2 e + h) 64 + L, so that each wave instruction writes or reads one contiguous
// kilobyte.  The aggregates are carried between segments without any rounding.
__device__ __forceinline__ f32x4 *slot_piece(float *S, int e, int h, int L) {
    return reinterpret_cast<f32x4 *>(S) + (2 * e + h) * 64 + L;
}
__device__ __forceinline__ const f32x4 *slot_piece(const float *S, int e, int h, int L) {
    return reinterpret_cast<const f32x4 *>(S) + (2 * e + h) * 64 + L;
}

// Position of feature f in a row-major feature tile.  With PERM, each 32-feature group is
// stored in the K order of two stacked accumulator blocks (lane group g reads features
// {4g..4g+3, 16+4g..16+4g+3} as one 16-byte run), so the read-out operand that pairs with
// the carried state is one 16-byte LDS read.  The scores read both feature tiles in the
// same physical order, a consistent permutation of their contraction index.  Four
// consecutive features (f0 % 4 == 0) stay contiguous.
template <bool PERM>
__device__ __forceinline__ int feat_pos(int f0) {
    if (!PERM) return f0;
    const int fl = f0 & 31;
    return (f0 & ~31) + 8 * ((fl & 15) >> 2) + ((fl & 16) ? 4 : 0);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// 16 bytes from an 8-byte-aligned LDS address, as two 8-byte reads.
__device__ __forceinline__ bf16x8 load8_as_halves(const bf16_t *p) { return cat(load4(p), load4(p + 4)); }

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i
// receives, in slot s, element (i % 4) of the 4-element run addressed by lane 4 s + i / 4.
// Pointing lane i of a group at row (r0 + i / 4), columns (c0 + 4 (i % 4)) .. +3 of a
// row-major tile therefore hands lane i column c0 + i, rows r0 .. r0+3: one half of an MFMA
// operand whose K index runs down the tile's rows.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16_t *p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// MFMA operand from a row-major tile by two transposing reads: lane (column c0 + r16,
// K rows r0 + 8 g .. r0 + 8 g + 7).  `lane_off` = (8 g + r16 / 4) * stride + 4 * (r16 % 4) is
// the per-lane part of the address; `koff` = r0 * stride + (position of column c0), a
// compile-time constant in every caller, so the reads use immediate offsets.
__device__ __forceinline__ bf16x8 operand_down_rows(const bf16_t *tile, int lane_off, int koff, int stride) {
    const bf16_t *p = tile + lane_off + koff;
    return cat(lds_read_tr(p), lds_read_tr(p + 4 * stride));
}


// Physical position of the 16-feature block k's first column in a permuted feature tile
// (columns of block k are at this position + 8 q + r for q = 0..3, r = 0..3).
__device__ __forceinline__ constexpr int perm_block_pos(int k) { return 32 * (k >> 1) + 4 * (k & 1); }

// Stored position of 16-byte granule G of row r in a [rows][D] bf16 staging tile, and its
// inverse.  256-byte rows are rotated by 2 r granules, so that 16 rows x 4 consecutive
// granules read together fall on the bank pattern of a 32-byte row pitch; shorter rows are
// XOR-swizzled.
template <int D>
__device__ __forceinline__ int stage_pos(int r, int G) {
    constexpr int NG = D / 8, NSW = NG < 8 ? NG : 8;
    if (NG == 16) return (G + 2 * r) & 15;
    return G ^ (r % NSW);
}
template <int D>
__device__ __forceinline__ int stage_granule(int r, int P) {
    constexpr int NG = D / 8, NSW = NG < 8 ? NG : 8;
    if (NG == 16) return (P - 2 * r) & 15;
    return P ^ (r % NSW);
}

// Value column held by MFMA column c (0..15) of value block vb of the wave with value part nq.
// The VB blocks of a wave interleave in runs of four, so that a lane of a transposed
// accumulator (rows = value columns 4 g .. 4 g + 3 of each block) holds the 4 VB contiguous
// columns 16 VB nq + 4 VB g .. +4 VB - 1 of one token.  The V tile in LDS stores value column
// value_col(nq, vb, c) at position 16 VB nq + 16 vb + c, so each block's operand is read from
// 16 contiguous positions.
template <int VB>
__device__ __forceinline__ constexpr int value_col(int nq, int vb, int c) {
    return 16 * VB * nq + 4 * VB * (c >> 2) + 4 * vb + (c & 3);
}

// Eight consecutive value columns n0 .. n0 + 7 (n0 % 8 == 0) of one token into row `row` of
// the V tile, at the positions value_col implies.
template <int VB>
__device__ __forceinline__ void store_v8(bf16_t *row, int n0, const bf16x8 &v) {
    if (VB == 1) {
        store8(row + n0, v);
    } else {  // VB == 2: columns 8 m .. 8 m + 7 of a 32-column group are runs m of blocks 0 and 1
        const int grp = n0 & ~31, m = (n0 & 31) >> 3;
        store4(row + grp + 4 * m, __builtin_shufflevector(v, v, 0, 1, 2, 3));
        store4(row + grp + 16 + 4 * m, __builtin_shufflevector(v, v, 4, 5, 6, 7));
    }
}

// Normalised outputs of one chunk kept in registers until the next chunk is under way, so
// that the wait for the next chunk's loads does not also wait for these stores to retire.
template <int D, int C>
struct PendingY {
    bf16x4 v[WideCfg<D, C>::IBF][WideCfg<D, C>::VB];
};

// Loads of the next chunk, issued one chunk ahead: q and k go straight into LDS staging
// tiles (global_load_lds), V into a few registers.
// Stored position of granule G of row r in a two-buffer V tile (256-byte rows): rotated by 4
// per row, so that the transposing reads of four rows x four 16-byte-spaced runs hit 16
// distinct granules.
__device__ __forceinline__ int v_pos(int r, int G) { return (G + 4 * r) & 15; }

template <int D, int C>
struct Prefetch {
    bf16x8 vp[WideCfg<D, C>::VPT];
};

// 16 bytes per lane from global memory straight into LDS (lane l -> lds_dst + 16 l), through
// M0.  Written as inline assembly on purpose: the compiler then does not track these LDS writes
// and does not stall every later LDS read until they land (it cannot tell the target buffers
// apart).  Callers make the data visible themselves: s_waitcnt vmcnt(0), then a barrier.  The
// hidden loads only make the compiler's own vmcnt waits more conservative (loads retire in
// order), never less.
__device__ __forceinline__ void load_to_lds_16(const void *gsrc, void *lds_dst_uniform) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds_dst_uniform));
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gsrc), "s"(lds) : "m0");
}

// The same from a uniform base address (SGPRs) plus a 32-bit per-lane byte offset, so that the
// per-chunk address is one scalar add instead of per-lane 64-bit arithmetic.
__device__ __forceinline__ void load_to_lds_16s(const void *sbase, uint32_t voff, void *lds_dst_uniform) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds_dst_uniform));
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds)
                 : "m0");
}

// s_waitcnt immediates (gfx9 layout: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8):
// LDS operations finished and at most `vm` vector memory operations outstanding.
constexpr int waitcnt_lds_vm(int vm) { return (vm & 15) | (7 << 4) | (0 << 8) | (((vm >> 4) & 3) << 14); }

// Per-lane source offsets of the direct loads of [C][128] bf16 tiles by 8 waves (wave w moves
// 1 KB blocks w, w + 8, ...): byte offsets within the tile's rows for the q / k staging layout
// (stage_pos) and the V layout (v_pos), and the row.  A lane whose row lies past the end reads
// the same granule of row 0 (x0, v0): the row is then a copy of row 0 in the tile's layout, so a
// non-finite value met by the row's zero features stays in its own value column.
template <int C>
struct DmaLanes128 {
    static constexpr int NB = C / 32;
    uint32_t ox[NB], ov[NB], x0[NB], v0[NB];
    int row[NB];
    __device__ __forceinline__ DmaLanes128(int w, int lane) {
#pragma unroll
        for (int bb = 0; bb < NB; bb++) {
            const int slot = 64 * (w + 8 * bb) + lane;
            const int r = slot / 16, P = slot % 16;
            row[bb] = r;
            const int gx = stage_granule<128>(r, P), gv = (P - 4 * r) & 15;
            ox[bb] = 2 * (r * 128 + 8 * gx);
            ov[bb] = 2 * (r * 128 + 8 * gv);
            x0[bb] = 16 * gx;
            v0[bb] = 16 * gv;
        }
    }
    // tile rows t0 .. t0 + C - 1 of x (valid of them) into `stage`, q / k layout or V layout
    template <bool V>
    __device__ __forceinline__ void issue(const bf16_t *x, int t0, int valid, int w, unsigned char *stage) const {
        const bf16_t *src = x + (size_t)t0 * 128;
#pragma unroll
        for (int bb = 0; bb < NB; bb++)
            load_to_lds_16s(src, row[bb] < valid ? (V ? ov[bb] : ox[bb]) : (V ? v0[bb] : x0[bb]),
                            stage + 1024 * (w + 8 * bb));
    }
};

// One [C][D] tile of x into its staging area: wave w moves blocks w, w + NW, ...; lane l of
// block b lands at slot 64 b + l = (row r, stored position P), which holds granule
// stage_granule(r, P).  Rows past the end read a valid row (their values are never used).
template <int D, int C>
__device__ __forceinline__ void stage_x(const bf16_t *__restrict__ x, int t0, int valid, int w, int lane,
                                        unsigned char *stage) {
    using K = WideCfg<D, C>;
#pragma unroll
    for (int bb = 0; bb < K::XBLK / K::NW; bb++) {
        const int blk = w + bb * K::NW;
        const int slot = 64 * blk + lane;
        const int r = slot / K::NG, P = slot % K::NG;
        const int kg = stage_granule<D>(r, P);
        const int rr = r < valid ? r : 0;
        load_to_lds_16(x + (size_t)(t0 + rr) * D + 8 * kg, stage + 1024 * blk);
    }
}

// One [C][D] tile of V into a two-buffer V tile (positions v_pos); rows past the end read a
// valid row: their keys' features are exactly zero, so they contribute nothing.
template <int D, int C>
__device__ __forceinline__ void stage_v(const bf16_t *__restrict__ v, int t0, int valid, int w, int lane,
                                        unsigned char *tile) {
    using K = WideCfg<D, C>;
#pragma unroll
    for (int bb = 0; bb < K::XBLK / K::NW; bb++) {
        const int blk = w + bb * K::NW;
        const int slot = 64 * blk + lane;
        const int r = slot / K::NG, P = slot % K::NG;
        const int G = (P - 4 * r) & 15;
        const int rr = r < valid ? r : 0;
        load_to_lds_16(v + (size_t)(t0 + rr) * D + 8 * G, tile + 1024 * blk);
    }
}

// Loads of one chunk into staging buffer BUF: q and k (and, with two buffers, V) straight into
// LDS, otherwise V into registers.
template <int D, int C, int MODE, int BUF>
__device__ __forceinline__ void issue_loads(Prefetch<D, C> &pf, const WideParams &p, size_t base, int t0, int valid,
                                            int w, int lane, int tid, unsigned char *smem) {
    using K = WideCfg<D, C, MODE>;
    if (MODE != WM_STATE) stage_x<D, C>(p.q + base, t0, valid, w, lane, smem + K::OFF_XQ + BUF * K::SZ_X);
    if (MODE != WM_READOUT) {
        stage_x<D, C>(p.k + base, t0, valid, w, lane, smem + K::OFF_XK + BUF * K::SZ_X);
        if (K::NBUF == 2) {
            stage_v<D, C>(p.v + base, t0, valid, w, lane, smem + K::OFF_V + BUF * K::SZ_V1);
            return;
        }
        constexpr int NC = D / 8;
#pragma unroll
        for (int it = 0; it < K::VPT; it++) {
            const int t = tid + it * K::NT;
            const int j = t / NC, nc = t % NC;
            pf.vp[it] = j < valid ? load8(p.v + base + (size_t)(t0 + j) * D + 8 * nc) : zero_bf16x8();
        }
    }
}

// x operand for the feature map (B operand: lane column = token i, K = input dim) from a
// staging tile.
template <int D>
__device__ __forceinline__ bf16x8 staged_x_operand(const unsigned char *stage, int i, int ks, int g) {
    using K = WideCfg<D>;
    const int kg = 4 * ks + g;
    if (8 * kg >= D) return zero_bf16x8();
    return *reinterpret_cast<const bf16x8 *>(stage + 16 * (i * K::NG + stage_pos<D>(i, kg)));
}

// Feature map of one chunk for this wave's directions and token blocks from prefetched x,
// written row-major (features contiguous, position feat_pos) into LDS.
template <int D, int C, bool IS_KEY, bool FULL, bool PERM = true>
__device__ __forceinline__ void phi_chunk(const unsigned char *stage, int valid,
                                          const bf16x8 (&wA)[WideCfg<D>::LB][WideCfg<D>::KSD],
                                          const float (&bl2)[WideCfg<D>::LB][4], int th, int dq, int g, int r16,
                                          bf16_t *sRow, int stride) {
    using K = WideCfg<D, C>;
#pragma unroll
    for (int ibl = 0; ibl < K::IBT; ibl++) {
        const int i = 16 * (th * K::IBT + ibl) + r16;
        bf16x8 xb[K::KSD];
#pragma unroll
        for (int ks = 0; ks < K::KSD; ks++) xb[ks] = staged_x_operand<D>(stage, i, ks, g);
        // With PERM, direction blocks 2 j and 2 j + 1 of a lane land in one 16-byte run
        // (positions 8 g .. 8 g + 7 of their 32-feature group): write them together where the
        // tile pitch allows 16-byte stores.
        constexpr bool PAIR = PERM && !IS_KEY && K::LB % 2 == 0;
        bf16x4 pe[K::LB], ne[K::LB];
#pragma unroll
        for (int mb = 0; mb < K::LB; mb++) {
            f32x4 a = zero4();
#pragma unroll
            for (int ks = 0; ks < K::KSD; ks++) a = mfma_bf16(wA[mb][ks], xb[ks], a);
            // a: lane holds u for token i and directions fb4 .. fb4 + 3
            f32x4 ep, en;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float u = a[r] * kLog2e + bl2[mb][r];
                ep[r] = exp2_fast(u);
                en[r] = exp2_fast(-u);
            }
            if (IS_KEY && !FULL && i >= valid) {  // keys past the end contribute nothing
                ep = zero4();
                en = zero4();
            }
            pe[mb] = to_bf16x4(ep);
            ne[mb] = to_bf16x4(en);
        }
#pragma unroll
        for (int mb = 0; mb < K::LB; mb++) {
            const int fb4 = dq * K::DPW + 16 * mb + 4 * g;
            if (PAIR) {
                if (mb % 2 == 0) {
                    store8(sRow + i * stride + feat_pos<PERM>(fb4), cat(pe[mb], pe[mb + 1]));
                    store8(sRow + i * stride + feat_pos<PERM>(D + fb4), cat(ne[mb], ne[mb + 1]));
                }
            } else {
                store4(sRow + i * stride + feat_pos<PERM>(fb4), pe[mb]);
                store4(sRow + i * stride + feat_pos<PERM>(D + fb4), ne[mb]);
            }
        }
    }
}

// Directions of direction group dq as MFMA A operands: row l = dq DPW + 16 mb + r16, K = input
// dim; bias pre-multiplied by log2(e) for the accumulator rows l = dq DPW + 16 mb + 4 g + r.
template <int D>
__device__ __forceinline__ void load_directions(const bf16_t *__restrict__ W, const bf16_t *__restrict__ b, int h,
                                                int dq, int g, int r16,
                                                bf16x8 (&wA)[WideCfg<D>::LB][WideCfg<D>::KSD],
                                                float (&bl2)[WideCfg<D>::LB][4]) {
    using K = WideCfg<D>;
    const bf16_t *Wh = W + (size_t)h * D * D;
#pragma unroll
    for (int mb = 0; mb < K::LB; mb++) {
        const int l = dq * K::DPW + 16 * mb + r16;
#pragma unroll
        for (int ks = 0; ks < K::KSD; ks++) {
            const int m0 = 32 * ks + 8 * g;
            wA[mb][ks] = (m0 < D) ? load8(Wh + (size_t)l * D + m0) : zero_bf16x8();
        }
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int lb = dq * K::DPW + 16 * mb + 4 * g + r;
            bl2[mb][r] = b ? bf16_bits_to_float(b[(size_t)h * D + lb]) * kLog2e : 0.0f;
        }
    }
}

// Per-head W (d = 128) into LDS by direct loads, in the layout of stage_w: a [128][128] tile
// staged like the x tiles (8 waves, four 1 KB blocks each).
__device__ __forceinline__ void stage_w_dma128(const bf16_t *__restrict__ W, int h, int w, int lane, unsigned char *sW) {
    const DmaLanes128<128> wl(w, lane);
    wl.issue<false>(W + (size_t)h * 128 * 128, 0, 128, w, sW);
}

// Per-head W into LDS (swizzled like the x tiles), once per workgroup.
template <int D>
__device__ __forceinline__ void stage_w(const bf16_t *__restrict__ W, int h, int tid, unsigned char *sW) {
    using K = WideCfg<D>;
    const bf16_t *Wh = W + (size_t)h * D * D;
    for (int t = tid; t < D * K::NG; t += K::NT) {
        const int l = t / K::NG, kg = t % K::NG;
        *reinterpret_cast<bf16x8 *>(sW + 16 * (l * K::NG + stage_pos<D>(l, kg))) = load8(Wh + (size_t)l * D + 8 * kg);
    }
}

// This wave's directions as MFMA A operands from the staged W.
template <int D>
__device__ __forceinline__ void load_w_operands(const unsigned char *sW, int dq, int g, int r16,
                                                bf16x8 (&wA)[WideCfg<D>::LB][WideCfg<D>::KSD]) {
    using K = WideCfg<D>;
#pragma unroll
    for (int mb = 0; mb < K::LB; mb++) {
        const int l = dq * K::DPW + 16 * mb + r16;
#pragma unroll
        for (int ks = 0; ks < K::KSD; ks++) {
            const int kg = 4 * ks + g;
            wA[mb][ks] = (8 * kg < D) ? *reinterpret_cast<const bf16x8 *>(sW + 16 * (l * K::NG + stage_pos<D>(l, kg)))
                                      : zero_bf16x8();
        }
    }
}

// Bias of this wave's directions, times log2(e), for the accumulator rows dq DPW + 16 mb + 4 g + r.
template <int D>
__device__ __forceinline__ void load_bias(const bf16_t *__restrict__ b, int h, int dq, int g,
                                          float (&bl2)[WideCfg<D>::LB][4]) {
    using K = WideCfg<D>;
    // one test of the pointer around all the loads: tested per element, each load would sit
    // in its own branch and be waited for before the next is issued
    if (b) {
#pragma unroll
        for (int mb = 0; mb < K::LB; mb++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                bl2[mb][r] = bf16_bits_to_float(b[(size_t)h * D + dq * K::DPW + 16 * mb + 4 * g + r]) * kLog2e;
    } else {
#pragma unroll
        for (int mb = 0; mb < K::LB; mb++)
#pragma unroll
            for (int r = 0; r < 4; r++) bl2[mb][r] = 0.0f;
    }
}

// Intra-chunk score task of wave w (query block ib, key blocks jlo..jhi, row-sum slot).
// Every (query block, key block <= it) pair is covered exactly once; tasks with an empty
// key range still write zero row sums for their slot.
template <int NW, int NCB>
__device__ __forceinline__ bool score_task(int w, int qq, int &ib, int &jlo, int &jhi, int &slot) {
    if (NW == 8 && NCB == 2) {  // (0,0) (1,0) (1,1), plus the empty (0, slot 1)
        if (w >= 4 || qq > 0) return false;
        ib = (w == 1 || w == 2) ? 1 : 0;
        jlo = (w == 2) ? 1 : 0;
        jhi = (w == 3) ? -1 : (w == 2 ? 1 : 0);
        slot = (w >= 2) ? 1 : 0;
        return true;
    }
    if (NW == 8) {
        // NCB == 4: the 10 (query, key) block pairs in tasks of one or two pairs, balanced over
        // the SIMDs (waves w and w + 4 share one); waves 6 and 7 only clear row-sum slots.
        static_assert(NW != 8 || NCB == 4 || NCB == 2, "8-wave split expects 32- or 64-token chunks");
        constexpr int T_IB[8] = {0, 1, 2, 3, 3, 2, 0, 1};
        constexpr int T_LO[8] = {0, 0, 0, 2, 0, 2, 0, 0};
        constexpr int T_HI[8] = {0, 1, 1, 3, 1, 2, -1, -1};
        constexpr int T_SL[8] = {0, 0, 0, 1, 0, 1, 1, 1};
        if (qq > 0) return false;
        ib = T_IB[w];
        jlo = T_LO[w];
        jhi = T_HI[w];
        slot = T_SL[w];
        return true;
    }
    constexpr int PER = NCB / NW;
    if (qq >= PER) return false;
    ib = w * PER + qq;
    jlo = 0;
    jhi = ib;
    slot = 0;
    return true;
}

// Stores the normalised outputs of one chunk: lane (g, r16) holds token 16 ib + r16 of the
// chunk, value columns value_col(nq, vb, 4 g + r) -- 4 VB contiguous values.
template <int D, int C, bool FULL>
__device__ __forceinline__ void store_y(bf16_t *__restrict__ y, size_t base, int t0, int valid, const PendingY<D, C> &py,
                                        int fa, int nq, int g, int r16) {
    using K = WideCfg<D, C>;
#pragma unroll
    for (int ibo = 0; ibo < K::IBF; ibo++) {
        const int i = 16 * (fa * K::IBF + ibo) + r16;
        if (!FULL && i >= valid) continue;
        bf16_t *dst = y + base + (size_t)(t0 + i) * D + value_col<K::VB>(nq, 0, 4 * g);
        if (K::VB == 2)
            store8(dst, cat(py.v[ibo][0], py.v[ibo][K::VB - 1]));
        else
            store4(dst, py.v[ibo][0]);
    }
}

template <int D, int C, int MODE, bool FULL, int BUF>
__device__ __forceinline__ void chunk_step(const WideParams &p, size_t base, int t0, int valid, int t_next,
                                           int valid_next, unsigned char *smem, Prefetch<D, C> &pf,
                                           const float (&bl2)[WideCfg<D>::LB][4],
                                           f32x4 (&sacc)[WideCfg<D>::FBW][WideCfg<D>::VB],
                                           f32x4 (&zacc)[WideCfg<D>::ZB], PendingY<D, C> &py, int t_pending,
                                           const bf16x8 (&wA)[WideCfg<D>::LB][WideCfg<D>::KSD], int tid) {
    using K = WideCfg<D, C, MODE>;
    bf16_t *sPQ = reinterpret_cast<bf16_t *>(smem + K::OFF_PQ);
    bf16_t *sPK = reinterpret_cast<bf16_t *>(smem + K::OFF_PK);
    bf16_t *sV = reinterpret_cast<bf16_t *>(smem + K::OFF_V + BUF * K::SZ_V1);
    bf16_t *sA = reinterpret_cast<bf16_t *>(smem + K::OFF_A);
    float *sDen = reinterpret_cast<float *>(smem + K::OFF_DEN);
    float *sX = reinterpret_cast<float *>(smem + K::OFF_PQ);  // phi(q) is dead once the read-out is done
    // wave index as a scalar: role branches on it stay scalar (never exec-masked around MFMAs)
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int th = w / K::NDQ, dq = w % K::NDQ;  // feature-map role
    const int fa = w / K::NN, nq = w % K::NN;     // state role: feature part, value part

    // two buffers: the next chunk's inputs go into the other one right away
    if (K::NBUF == 2 && valid_next > 0)
        issue_loads<D, C, MODE, BUF ^ 1>(pf, p, base, t_next, valid_next, w, lane, tid, smem);
    // outputs of the previous chunk
    if (MODE != WM_STATE && t_pending >= 0) store_y<D, C, true>(p.y, base, t_pending, K::C, py, fa, nq, g, r16);

    // ---- phase 1: (V and) feature maps into LDS
    if (MODE != WM_READOUT) {
        if (K::NBUF == 1) {
            constexpr int NC = D / 8;
#pragma unroll
            for (int it = 0; it < K::VPT; it++) {
                const int t = tid + it * K::NT;
                store_v8<K::VB>(sV + (t / NC) * K::RV, 8 * (t % NC), pf.vp[it]);
            }
        }
        phi_chunk<D, C, true, FULL>(smem + K::OFF_XK + BUF * K::SZ_X, valid, wA, bl2, th, dq, g, r16, sPK, K::RK);
    }
    if (MODE != WM_STATE)
        phi_chunk<D, C, false, FULL>(smem + K::OFF_XQ + BUF * K::SZ_X, valid, wA, bl2, th, dq, g, r16, sPQ, K::RQ);
    __syncthreads();
    // one buffer: it is free again, start moving the next chunk in
    if (K::NBUF == 1 && valid_next > 0)
        issue_loads<D, C, MODE, 0>(pf, p, base, t_next, valid_next, w, lane, tid, smem);

    // Read-out accumulators are transposed: numT[ib][vb] holds, in lane (g, r16), token
    // 16 ib + r16 and value columns value_col(nq, vb, 4 g + r).
    f32x4 numT[K::NCB][K::VB];
    if (MODE != WM_STATE) {
        // ---- phase 2: intra-chunk scores, read-out against the carried state, denominators
        if (MODE == WM_CAUSAL) {
#pragma unroll
            for (int qq = 0; qq < K::NCB; qq++) {
                int ib = 0, jlo = 0, jhi = -1, slot = 0;
                if (!score_task<K::NW, K::NCB>(w, qq, ib, jlo, jhi, slot)) continue;
                constexpr int MAXJ = K::NW == 8 ? (K::NCB == 2 ? 1 : 2) : K::NCB;
                f32x4 a[MAXJ];
#pragma unroll
                for (int jj = 0; jj < MAXJ; jj++) a[jj] = zero4();
                if (jlo <= jhi) {
#pragma unroll
                    for (int ks = 0; ks < K::KSF; ks++) {
                        const bf16x8 qb = load8(sPQ + (16 * ib + r16) * K::RQ + 32 * ks + 8 * g);
#pragma unroll
                        for (int jj = 0; jj < MAXJ; jj++)
                            if (jlo + jj <= jhi)
                                a[jj] = mfma_bf16(load8_as_halves(sPK + (16 * (jlo + jj) + r16) * K::RK + 32 * ks + 8 * g),
                                                  qb, a[jj]);
                    }
                }
                float rs = 0.0f;
#pragma unroll
                for (int jj = 0; jj < MAXJ; jj++) {
                    const int jb = jlo + jj;
                    if (jb > jhi) continue;
                    // a = A^T[j][i]: lane holds i = 16 ib + r16, j = 16 jb + 4 g + r; keep j <= i
                    f32x4 av = a[jj];
                    if (jb == ib) {
#pragma unroll
                        for (int r = 0; r < 4; r++)
                            if (4 * g + r > r16) av[r] = 0.0f;
                    }
                    const bf16x4 ab = to_bf16x4(av);
                    rs += ((float)ab[0] + (float)ab[1]) + ((float)ab[2] + (float)ab[3]);
                    store4(sA + (16 * ib + r16) * K::RA + 16 * jb + 4 * g, ab);
                }
                if (jlo == 0 && (ib & 1) == 0 && ib + 1 < K::NCB) {  // the K step over block ib also covers ib + 1
                    bf16x4 zz;
                    zz[0] = zz[1] = zz[2] = zz[3] = (__bf16)0.0f;
                    store4(sA + (16 * ib + r16) * K::RA + 16 * (ib + 1) + 4 * g, zz);
                }
                rs += __shfl_xor(rs, 16);
                rs += __shfl_xor(rs, 32);
                if (g == 0) sDen[(K::NW + slot) * K::C + 16 * ib + r16] = rs;
            }
        }
#pragma unroll
        for (int ib = 0; ib < K::NCB; ib++)
#pragma unroll
            for (int vb = 0; vb < K::VB; vb++) numT[ib][vb] = zero4();
#pragma unroll
        for (int kk = 0; kk < K::KSW; kk++) {
            const int ks = fa * K::KSW + kk;
            bf16x8 sb[K::VB];
#pragma unroll
            for (int vb = 0; vb < K::VB; vb++) sb[vb] = acc_pair_to_operand(sacc[2 * kk][vb], sacc[2 * kk + 1][vb]);
#pragma unroll
            for (int ib = 0; ib < K::NCB; ib++) {
                const bf16x8 qop = load8(sPQ + (16 * ib + r16) * K::RQ + 32 * ks + 8 * g);
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++) numT[ib][vb] = mfma_bf16(sb[vb], qop, numT[ib][vb]);
            }
        }
        {  // partial denominators over this wave's z rows (K step w of the features)
            const bf16x8 zb = acc_pair_to_operand(zacc[0], zacc[1]);
#pragma unroll
            for (int ib = 0; ib < K::NCB; ib++) {
                const f32x4 dacc = mfma_bf16(zb, load8(sPQ + (16 * ib + r16) * K::RQ + 32 * w + 8 * g), zero4());
                if (g == 0) sDen[w * K::C + 16 * ib + r16] = dacc[0];
            }
        }
        if (K::NF == 2) {
            __syncthreads();  // every wave is done with the phi(q) tile: reuse it for the exchange
#pragma unroll
            for (int ib = 0; ib < K::NCB; ib++) {
                if (ib / K::IBF == fa) continue;
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++)
                    *reinterpret_cast<f32x4 *>(sX + (16 * ib + r16) * K::XS + value_col<K::VB>(nq, vb, 4 * g)) =
                        numT[ib][vb];
            }
        }
    }
    __syncthreads();

    // ---- phase 3: exchange, intra-chunk product, output, state update
    // V operands: lane column c <-> value column value_col(nq, vb, c), K = tokens
    bf16x8 vop[K::KSC][K::VB];
    if (MODE != WM_READOUT) {
        if (K::NBUF == 2) {
            // rows 8 g + r16 / 4 (+4, +32 ks keep the rotation), runs of 4 columns 16 bytes apart:
            // granule 4 nq + r16 % 4, byte 8 vb of it
            const int r0 = 8 * g + (r16 >> 2);
            const int lane_v = r0 * K::RV + 8 * v_pos(r0, 4 * nq + (r16 & 3));
#pragma unroll
            for (int ks = 0; ks < K::KSC; ks++)
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++)
                    vop[ks][vb] = operand_down_rows(sV, lane_v, 32 * ks * K::RV + 4 * vb, K::RV);
        } else {
            const int lane_v = (8 * g + (r16 >> 2)) * K::RV + 4 * (r16 & 3) + 16 * nq * K::VB;
#pragma unroll
            for (int ks = 0; ks < K::KSC; ks++)
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++)
                    vop[ks][vb] = operand_down_rows(sV, lane_v, 32 * ks * K::RV + 16 * vb, K::RV);
        }
    }
    if (MODE != WM_STATE) {
#pragma unroll
        for (int ib = 0; ib < K::NCB; ib++) {
            if (ib / K::IBF != fa) continue;  // rows finalised by the other feature part
            const int i = 16 * ib + r16;
            if (K::NF == 2) {
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++)
                    numT[ib][vb] += *reinterpret_cast<const f32x4 *>(sX + i * K::XS + value_col<K::VB>(nq, vb, 4 * g));
            }
            if (MODE == WM_CAUSAL) {
#pragma unroll
                for (int ks = 0; ks <= ib / 2; ks++) {
                    const bf16x8 a = load8(sA + i * K::RA + 32 * ks + 8 * g);
#pragma unroll
                    for (int vb = 0; vb < K::VB; vb++) numT[ib][vb] = mfma_bf16(vop[ks][vb], a, numT[ib][vb]);
                }
            }
            float den = 0.0f;
#pragma unroll
            for (int pw = 0; pw < K::NW + (MODE == WM_CAUSAL ? K::NJ : 0); pw++) den += sDen[pw * K::C + i];
            const float rden = __builtin_amdgcn_rcpf(den);
#pragma unroll
            for (int vb = 0; vb < K::VB; vb++) {
                f32x4 o;
#pragma unroll
                for (int r = 0; r < 4; r++) o[r] = numT[ib][vb][r] * rden;
                py.v[ib % K::IBF][vb] = to_bf16x4(o);
            }
        }
        // full chunks: stored during the next chunk; the last, partial chunk: now
        if (!FULL) store_y<D, C, false>(p.y, base, t0, valid, py, fa, nq, g, r16);
    }
    if (MODE != WM_READOUT) {
        const bf16x8 ones = ones_bf16x8();
        // features of block k sit at perm_block_pos(k) + 8 q + r: lane q = r16 % 4 reads run q
        const int lane_k = (8 * g + (r16 >> 2)) * K::RK + 8 * (r16 & 3);
        const bf16_t *sPKf = sPK + perm_block_pos(fa * K::FBW);   // fa * FBW is even
        const bf16_t *sPKz = sPK + perm_block_pos(w * K::ZB);     // w * ZB is even
#pragma unroll
        for (int ks = 0; ks < K::KSC; ks++) {
#pragma unroll
            for (int fb = 0; fb < K::FBW; fb++) {
                const bf16x8 a = operand_down_rows(sPKf, lane_k, 32 * ks * K::RK + perm_block_pos(fb), K::RK);
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++) sacc[fb][vb] = mfma_bf16(a, vop[ks][vb], sacc[fb][vb]);
            }
#pragma unroll
            for (int zb = 0; zb < K::ZB; zb++) {
                const bf16x8 a = operand_down_rows(sPKz, lane_k, 32 * ks * K::RK + perm_block_pos(zb), K::RK);
                zacc[zb] = mfma_bf16(a, ones, zacc[zb]);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the next chunk's direct loads have landed in LDS
    __syncthreads();
}

// Tokens per chunk: for d = 128 the causal pass takes 32-token chunks (its registers and
// scores balance better), the other passes 64.
constexpr int wide_chunk(int D, int MODE) { return (D == 128 && MODE == WM_CAUSAL) ? 32 : 64; }

// One workgroup's work: segment s of sequence bh, with `smem` the K::LDS_BYTES of its tiles.
template <int D, int MODE>
__device__ __forceinline__ void wide_body(const WideParams &p, unsigned char *smem, int bh, int s) {
    constexpr int C = wide_chunk(D, MODE);
    using K = WideCfg<D, C, MODE>;
    static_assert(K::LDS_BYTES <= 160 * 1024, "LDS budget");

    const int tid = threadIdx.x;
    // wave index as a scalar: role branches on it stay scalar (never exec-masked around MFMAs)
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int dq = w % K::NDQ;
    const int fa = w / K::NN, nq = w % K::NN;
    const int h = bh % p.H;
    const int t_begin = s * p.seg_len;
    const int t_end = min(p.N, t_begin + p.seg_len);
    const size_t base = (size_t)bh * p.N * D;

    Prefetch<D, C> pf;
    if (t_begin < t_end) issue_loads<D, C, MODE, 0>(pf, p, base, t_begin, min(K::C, t_end - t_begin), w, lane, tid, smem);

    float bl2[K::LB][4];
    load_bias<D>(p.b, h, dq, g, bl2);
    stage_w<D>(p.W, h, tid, smem + K::OFF_W);

    // State: S[f][n] for feature blocks fa*FBW .. and this wave's value columns; z rows of
    // feature blocks w*ZB .. (every column of the z accumulator holds the same value).
    // Segment slots in the workspace hold S in fp32 in the register image of this layout:
    // accumulators k = fb VB + vb of lane `lane` in wave w are paired, the pair j = k / 2 being
    // slot piece w IMG8 + j (halves k0, k1), so that reading and writing a slot are whole 1 KB
    // rows per instruction.
    f32x4 sacc[K::FBW][K::VB];
    f32x4 zacc[K::ZB];
    {
        const float *Si = nullptr, *zi = nullptr;
        if (MODE != WM_STATE && p.S_in) {
            const size_t slot = (size_t)bh * p.in_bh_stride + (size_t)s * p.in_seg_stride;
            Si = p.S_in + slot * K::DP * D;
            zi = p.z_in + slot * K::DP;
        }
#pragma unroll
        for (int fb = 0; fb < K::FBW; fb++)
#pragma unroll
            for (int vb = 0; vb < K::VB; vb++) sacc[fb][vb] = zero4();
#pragma unroll
        for (int zb = 0; zb < K::ZB; zb++) zacc[zb] = zero4();
        if (Si) {
#pragma unroll
            for (int fb = 0; fb < K::FBW; fb++)
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++) {
                    const int n = value_col<K::VB>(nq, vb, r16);
#pragma unroll
                    for (int r = 0; r < 4; r++) sacc[fb][vb][r] = Si[(size_t)(16 * (fa * K::FBW + fb) + 4 * g + r) * D + n];
                }
#pragma unroll
            for (int zb = 0; zb < K::ZB; zb++)
#pragma unroll
                for (int r = 0; r < 4; r++) zacc[zb][r] = zi[16 * (w * K::ZB + zb) + 4 * g + r];
        }
        // slots added to the starting state: the exclusive prefix (slot_mode 1), the total
        // (slot_mode 2) or the earlier segments' aggregates, summed here (slot_mode 3)
        int t0 = 0, t1 = 0;
        if (MODE != WM_STATE && p.slot_mode == 1 && s > 0) t0 = s, t1 = s + 1;
        if (MODE != WM_STATE && p.slot_mode == 2) t0 = 0, t1 = 1;
        if (MODE != WM_STATE && p.slot_mode == 3) t0 = 0, t1 = s;
        for (int slot = t0; slot < t1; slot++) {
            const size_t sl = (size_t)bh * p.slot_bh_stride + slot;
            const float *img = p.S_slots + sl * K::DP * D;
            f32x4 t[K::IMG8][2];
#pragma unroll
            for (int j = 0; j < K::IMG8; j++)
#pragma unroll
                for (int hf = 0; hf < 2; hf++) t[j][hf] = *slot_piece(img, w * K::IMG8 + j, hf, lane);
            const float *zs = p.z_slots + sl * K::DP;
#pragma unroll
            for (int zb = 0; zb < K::ZB; zb++)
#pragma unroll
                for (int r = 0; r < 4; r++) zacc[zb][r] += zs[16 * (w * K::ZB + zb) + 4 * g + r];
#pragma unroll
            for (int j = 0; j < K::IMG8; j++) {
                const int k0 = 2 * j, k1 = 2 * j + 1;
                sacc[k0 / K::VB][k0 % K::VB] += t[j][0];
                sacc[k1 / K::VB][k1 % K::VB] += t[j][1];
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // this wave's directions stay in registers for the whole segment
    bf16x8 wA[K::LB][K::KSD];
    load_w_operands<D>(smem + K::OFF_W, dq, g, r16, wA);
    __syncthreads();  // the W tile is overwritten by the first chunk's features

    PendingY<D, C> py;
    int t0 = t_begin;
    auto prev = [&](int t) { return t > t_begin ? t - K::C : -1; };
    if (K::NBUF == 2) {
        // buffers alternate: chunk pairs, then at most one more full chunk and a partial one
        for (; t0 + 2 * K::C <= t_end; t0 += 2 * K::C) {
            chunk_step<D, C, MODE, true, 0>(p, base, t0, K::C, t0 + K::C, K::C, smem, pf, bl2, sacc, zacc, py,
                                            prev(t0), wA, tid);
            const int t1 = t0 + K::C;
            chunk_step<D, C, MODE, true, 1>(p, base, t1, K::C, t1 + K::C, min(K::C, t_end - t1 - K::C), smem, pf, bl2,
                                            sacc, zacc, py, prev(t1), wA, tid);
        }
        if (t0 + K::C <= t_end) {
            chunk_step<D, C, MODE, true, 0>(p, base, t0, K::C, t0 + K::C, min(K::C, t_end - t0 - K::C), smem, pf, bl2,
                                            sacc, zacc, py, prev(t0), wA, tid);
            t0 += K::C;
            if (t0 < t_end)
                chunk_step<D, C, MODE, false, 1>(p, base, t0, t_end - t0, t_end, 0, smem, pf, bl2, sacc, zacc, py,
                                                 prev(t0), wA, tid);
        } else if (t0 < t_end) {
            chunk_step<D, C, MODE, false, 0>(p, base, t0, t_end - t0, t_end, 0, smem, pf, bl2, sacc, zacc, py,
                                             prev(t0), wA, tid);
        }
    } else {
        for (; t0 + K::C <= t_end; t0 += K::C) {
            const int t_next = t0 + K::C;
            chunk_step<D, C, MODE, true, 0>(p, base, t0, K::C, t_next, min(K::C, t_end - t_next), smem, pf, bl2, sacc,
                                            zacc, py, prev(t0), wA, tid);
        }
        if (t0 < t_end)
            chunk_step<D, C, MODE, false, 0>(p, base, t0, t_end - t0, t_end, 0, smem, pf, bl2, sacc, zacc, py, prev(t0),
                                             wA, tid);
    }
    // the last chunk's outputs, unless it was partial (stored at once)
    if (MODE != WM_STATE && t_end > t_begin && (t_end - t_begin) % K::C == 0)
        store_y<D, C, true>(p.y, base, t_end - K::C, K::C, py, fa, nq, g, r16);

    // ---- segment end: publish the aggregate (STATE, register image) or the final state
    //      (CAUSAL, last segment, feature-major)
    if (MODE == WM_STATE) {
        const size_t slot = (size_t)bh * p.slot_bh_stride + s;
        float *img = p.S_slots + slot * K::DP * D;
#pragma unroll
        for (int j = 0; j < K::IMG8; j++) {
            const int k0 = 2 * j, k1 = 2 * j + 1;
            *slot_piece(img, w * K::IMG8 + j, 0, lane) = sacc[k0 / K::VB][k0 % K::VB];
            *slot_piece(img, w * K::IMG8 + j, 1, lane) = sacc[k1 / K::VB][k1 % K::VB];
        }
        float *zs = p.z_slots + slot * K::DP;
        if (r16 == 0) {
#pragma unroll
            for (int zb = 0; zb < K::ZB; zb++)
#pragma unroll
                for (int r = 0; r < 4; r++) zs[16 * (w * K::ZB + zb) + 4 * g + r] = zacc[zb][r];
        }
        return;
    }
    float *So = nullptr, *zo = nullptr;
    if (MODE == WM_CAUSAL && p.S_out && s == p.nseg_grid - 1) {
        So = p.S_out + (size_t)bh * K::DP * D;
        zo = p.z_out + (size_t)bh * K::DP;
    }
    if (So) {
#pragma unroll
        for (int fb = 0; fb < K::FBW; fb++)
#pragma unroll
            for (int vb = 0; vb < K::VB; vb++) {
                const int n = value_col<K::VB>(nq, vb, r16);
#pragma unroll
                for (int r = 0; r < 4; r++) So[(size_t)(16 * (fa * K::FBW + fb) + 4 * g + r) * D + n] = sacc[fb][vb][r];
            }
        if (r16 == 0) {
#pragma unroll
            for (int zb = 0; zb < K::ZB; zb++)
#pragma unroll
                for (int r = 0; r < 4; r++) zo[16 * (w * K::ZB + zb) + 4 * g + r] = zacc[zb][r];
        }
    }
}

template <int D, int MODE>
__global__ __launch_bounds__(WideCfg<D>::NT, WideCfg<D>::MIN_WG_PER_CU) void wide_kernel(WideParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[WideCfg<D, wide_chunk(D, MODE), MODE>::LDS_BYTES];
    int bh, s;
    wg_head_segment(p.nseg_grid, bh, s);
    wide_body<D, MODE>(p, smem, bh, s);
}

// ---------------------------------------------------------------------------------------
// Segment aggregates with symmetric waves (d = 64 and 128, 64-token chunks).  Wave w of the
// d / 16 waves owns feature blocks w (exp(+u) of directions 16 w .. 16 w + 15) and d / 16 + w
// (their exp(-u)): it computes those features for all tokens of the chunk with the tokens as
// the MFMA rows (x from LDS, W^T in registers), turns them into the A operands of its own
// state update straight from the accumulators, and adds phi(k)^T V and phi(k)^T 1 into its rows
// of S and z.  The key features never pass through LDS, and every wave has exponentials to
// issue.  The contraction over the chunk's tokens runs in the order the accumulators hold
// them: K index 8 g + s of K step kt is token 32 kt + 4 g + s (s < 4) or 32 kt + 16 + 4 g + s - 4;
// V is read in the same order.
template <int D>
struct StateSymCfg {
    static constexpr int C = 64, DP = 2 * D, NW = D / 16, NT = 64 * NW;
    static constexpr int NG = D / 8;                      // 16-byte granules per row
    static constexpr int KSD = D / 32;                    // K steps over the head dim
    static constexpr int VB = D / 16;                     // value blocks
    static constexpr int SZ_X = C * D * 2;                // k staging and V tile alike
    static constexpr int NB = 3;                          // staging buffers: chunk c + 2 loads during chunk c
    static constexpr int OFF_W = 0;                       // W [D][D], x-tile layout
    static constexpr int OFF_V = OFF_W + D * D * 2;       // V tiles (granules at ssy_vpos)
    static constexpr int OFF_XK = OFF_V + NB * SZ_X;      // k staging tiles
    static constexpr int LDS_BYTES = OFF_XK + NB * SZ_X;
    static constexpr int WG_PER_CU = D == 128 ? 1 : 2;
    static_assert(LDS_BYTES * WG_PER_CU <= 160 * 1024, "LDS budget");
};

// Stored position of granule G of row r in this kernel's V tiles: rotated by 64 bytes per row
// (d = 128) or 32 bytes per row (d = 64), so that the transposing reads of four rows fall in
// distinct banks; the rotation repeats every 4 rows.
template <int D>
__device__ __forceinline__ int ssy_vpos(int r, int G) {
    return D == 128 ? (G + 4 * r) & 15 : (G + 2 * r) & 7;
}

// Direct loads of [C][D] bf16 tiles by NWV waves (wave w moves 1 KB blocks w, w + NWV, ...):
// per-lane byte offsets within the tile for the q / k staging layout (stage_pos) and this
// kernel's V layout, and the row.  A lane whose row lies past the end reads the same granule of
// row 0 (offsets x0, v0), so such a row is a copy of row 0 in the tile's layout: its zero
// features then meet row 0's values column by column, and a non-finite value stays in its own
// value column.
template <int D, int C, int NWV>
struct DmaLanesT {
    static constexpr int NG = D / 8;
    static constexpr int NB = C * D * 2 / 1024 / NWV;
    uint32_t ox[NB], ov[NB], x0[NB], v0[NB];
    int row[NB];
    __device__ __forceinline__ DmaLanesT(int w, int lane) {
#pragma unroll
        for (int bb = 0; bb < NB; bb++) {
            const int slot = 64 * (w + NWV * bb) + lane;
            const int r = slot / NG, P = slot % NG;
            row[bb] = r;
            // granule G is stored at ssy_vpos(r, G): position P holds G = P - rotation
            const int gx = stage_granule<D>(r, P), gv = D == 128 ? ((P - 4 * r) & 15) : ((P - 2 * r) & 7);
            ox[bb] = 2 * (r * D + 8 * gx);
            ov[bb] = 2 * (r * D + 8 * gv);
            x0[bb] = 16 * gx;
            v0[bb] = 16 * gv;
        }
    }
    template <bool V>
    __device__ __forceinline__ void issue(const bf16_t *x, int t0, int valid, int w, unsigned char *stage) const {
        const bf16_t *src = x + (size_t)t0 * D;
#pragma unroll
        for (int bb = 0; bb < NB; bb++)
            load_to_lds_16s(src, row[bb] < valid ? (V ? ov[bb] : ox[bb]) : (V ? v0[bb] : x0[bb]),
                            stage + 1024 * (w + NWV * bb));
    }
};

// V operand of value block vb and token K step kt in the token order above: two transposing
// reads, rows 32 kt + 4 g .. + 3 and 32 kt + 16 + 4 g .. + 3.  lane_v[vb] addresses row
// 4 g + r16 / 4 of value columns 16 vb + 4 (r16 % 4) .. + 3; rows 16 and 32 further use the same
// granule positions.
template <int D>
__device__ __forceinline__ bf16x8 ssy_v_operand(const bf16_t *sV, int lane_v, int kt) {
    return cat(lds_read_tr(sV + lane_v + 32 * kt * D), lds_read_tr(sV + lane_v + (32 * kt + 16) * D));
}

// Maximum and sum over the 16 lanes of each lane group (lanes 16 g .. 16 g + 15), every lane
// receiving the result: two quad exchanges, then rotations by 4 and 8 within the row (DPP).
__device__ __forceinline__ float dpp_f(float v, int ctrl_sel) {
    const int x = __builtin_bit_cast(int, v);
    int y;
    switch (ctrl_sel) {
    case 0: y = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true); break;   // quad_perm [1,0,3,2]
    case 1: y = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true); break;   // quad_perm [2,3,0,1]
    case 2: y = __builtin_amdgcn_mov_dpp(x, 0x124, 0xF, 0xF, true); break;  // row_ror:4
    default: y = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true); break; // row_ror:8
    }
    return __builtin_bit_cast(float, y);
}
__device__ __forceinline__ int dpp_i(int x, int ctrl_sel) {
    switch (ctrl_sel) {
    case 0: return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);
    case 1: return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);
    case 2: return __builtin_amdgcn_mov_dpp(x, 0x124, 0xF, 0xF, true);
    default: return __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true);
    }
}
// The maximum on integers whose order is that of the floats (negative floats with their magnitude
// bits flipped), so that each step is one integer maximum with the lane exchange folded in.
__device__ __forceinline__ float row16_max(float v) {
    int k = __float_as_int(v);
    k ^= (k >> 31) & 0x7fffffff;
#pragma unroll
    for (int j = 0; j < 4; j++) k = max(k, dpp_i(k, j));
    k ^= (k >> 31) & 0x7fffffff;
    return __int_as_float(k);
}
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
    for (int k = 0; k < 4; k++) v += dpp_f(v, k);
    return v;
}

template <int D>
__device__ __forceinline__ void ssy_chunk(const unsigned char *xk, const bf16_t *sV, int valid,
                                          const bf16x8 (&wB)[StateSymCfg<D>::KSD], float bias2,
                                          const int (&lane_v)[StateSymCfg<D>::VB], const bf16x8 &ones,
                                          f32x4 (&sacc)[2][StateSymCfg<D>::VB], f32x4 (&zacc)[2], int g, int r16) {
    using S = StateSymCfg<D>;
    // u^T for the four token blocks: rows tokens 16 tb + 4 g + r, column direction 16 w + r16
    // (x operands of K step ks + 1 read during the products of step ks)
    bf16x8 xn[4], xc[4];
#pragma unroll
    for (int tb = 0; tb < 4; tb++) xn[tb] = staged_x_operand<D>(xk, 16 * tb + r16, 0, g);
    f32x4 u[4];
#pragma unroll
    for (int tb = 0; tb < 4; tb++) u[tb] = zero4();
#pragma unroll
    for (int ks = 0; ks < S::KSD; ks++) {
#pragma unroll
        for (int tb = 0; tb < 4; tb++) xc[tb] = xn[tb];
        if (ks + 1 < S::KSD) {
#pragma unroll
            for (int tb = 0; tb < 4; tb++) xn[tb] = staged_x_operand<D>(xk, 16 * tb + r16, ks + 1, g);
        }
#pragma unroll
        for (int tb = 0; tb < 4; tb++) u[tb] = mfma_bf16(xc[tb], wB[ks], u[tb]);
    }
    // V operands of the first K step while the exponentials run
    bf16x8 vo[S::VB];
#pragma unroll
    for (int vb = 0; vb < S::VB; vb++) vo[vb] = ssy_v_operand<D>(sV, lane_v[vb], 0);
    bf16x4 ep[4], en[4];
#pragma unroll
    for (int tb = 0; tb < 4; tb++) {
        f32x4 a, b;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const float x = u[tb][r] * kLog2e + bias2;
            a[r] = exp2_fast(x);
            b[r] = exp2_fast(-x);
            if (16 * tb + 4 * g + r >= valid) a[r] = b[r] = 0.0f;  // keys past the end add nothing
        }
        ep[tb] = to_bf16x4(a);
        en[tb] = to_bf16x4(b);
    }
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
        const bf16x8 ap = cat(ep[2 * kt], ep[2 * kt + 1]), an = cat(en[2 * kt], en[2 * kt + 1]);
#pragma unroll
        for (int vb = 0; vb < S::VB; vb++) {
            sacc[0][vb] = mfma_bf16(ap, vo[vb], sacc[0][vb]);
            sacc[1][vb] = mfma_bf16(an, vo[vb], sacc[1][vb]);
            if (kt == 0) vo[vb] = ssy_v_operand<D>(sV, lane_v[vb], 1);  // the second K step's, in place
        }
        zacc[0] = mfma_bf16(ap, ones, zacc[0]);
        zacc[1] = mfma_bf16(an, ones, zacc[1]);
    }
}

// One workgroup's work: the aggregate of segment s of sequence bh into slot bh slot_bh_stride + s,
// with `smem` the S::LDS_BYTES of its tiles.
template <int D>
__device__ __forceinline__ void state_sym_body(const WideParams &p, unsigned char *smem, int bh, int s) {
    using S = StateSymCfg<D>;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int h = bh % p.H;
    const int t_begin = s * p.seg_len;
    const int t_end = min(p.N, t_begin + p.seg_len);
    const size_t base = (size_t)bh * p.N * D;
    const int n = t_end > t_begin ? (t_end - t_begin + S::C - 1) / S::C : 0;
    const DmaLanesT<D, S::C, S::NW> dl(w, lane);
    auto valid_of = [&](int c) { return min(S::C, t_end - (t_begin + S::C * c)); };
    auto v_buf = [&](int b) { return reinterpret_cast<const bf16_t *>(smem + S::OFF_V + b * S::SZ_X); };
    auto x_buf = [&](int b) { return smem + S::OFF_XK + b * S::SZ_X; };

    {  // W into LDS by direct loads, x-tile layout
        const DmaLanesT<D, D, S::NW> wl(w, lane);
        wl.template issue<false>(p.W + (size_t)h * D * D, 0, D, w, smem + S::OFF_W);
    }
    // The chunks go last to first (the sum does not depend on the order): the segment's first
    // chunks are then the ones still in L2 when the chunked pass, which starts with them, begins.
    // Step c handles chunk n - 1 - c.
    auto chunk_of = [&](int c) { return n - 1 - c; };
    for (int c = 0; c < 2 && c < n; c++) {  // steps 0 and 1; the loop fetches two steps ahead
        const int cc = chunk_of(c);
        dl.template issue<false>(p.k + base, t_begin + S::C * cc, valid_of(cc), w, x_buf(c));
        dl.template issue<true>(p.v + base, t_begin + S::C * cc, valid_of(cc), w, smem + S::OFF_V + c * S::SZ_X);
    }
    // bias of this lane's direction 16 w + r16, times log2(e)
    const float bias2 = p.b ? bf16_bits_to_float(p.b[(size_t)h * D + 16 * w + r16]) * kLog2e : 0.0f;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // W^T as the B operand: lane column = direction 16 w + r16, K = input dims 32 ks + 8 g .. + 7
    bf16x8 wB[S::KSD];
    {
        const int l = 16 * w + r16;
#pragma unroll
        for (int ks = 0; ks < S::KSD; ks++)
            wB[ks] = *reinterpret_cast<const bf16x8 *>(smem + S::OFF_W + 16 * (l * S::NG + stage_pos<D>(l, 4 * ks + g)));
    }
    int lane_v[S::VB];
    {
        const int row = 4 * g + (r16 >> 2);
#pragma unroll
        for (int vb = 0; vb < S::VB; vb++)
            lane_v[vb] = row * D + 8 * ssy_vpos<D>(row, 2 * vb + ((r16 & 3) >> 1)) + 4 * (r16 & 1);
    }
    const bf16x8 ones = ones_bf16x8();
    f32x4 sacc[2][S::VB];  // [exp(+u), exp(-u)][value block]: rows 16 fb + 4 g + r, columns 16 vb + r16
    f32x4 zacc[2];
#pragma unroll
    for (int f = 0; f < 2; f++) {
#pragma unroll
        for (int vb = 0; vb < S::VB; vb++) sacc[f][vb] = zero4();
        zacc[f] = zero4();
    }
    for (int c = 0; c < n; c++) {
        const int b = c % S::NB;
        const bool ahead = c + 2 < n;
        if (ahead) {  // k and V of step c + 2 into the buffers step c - 1 used
            const int t = t_begin + S::C * chunk_of(c + 2), b2 = (c + 2) % S::NB;
            dl.template issue<false>(p.k + base, t, min(S::C, t_end - t), w, x_buf(b2));
            dl.template issue<true>(p.v + base, t, min(S::C, t_end - t), w, smem + S::OFF_V + b2 * S::SZ_X);
        }
        ssy_chunk<D>(x_buf(b), v_buf(b), valid_of(chunk_of(c)), wB, bias2, lane_v, ones, sacc, zacc, g, r16);
        // step c + 1's loads (issued a step ago) have landed; step c + 2's stay in flight
        if (ahead)
            __builtin_amdgcn_s_waitcnt(waitcnt_lds_vm(2 * DmaLanesT<D, S::C, S::NW>::NB));
        else
            __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // Slot s in the register image the chunked pass of the same d reads back.
    const size_t slot = (size_t)bh * p.slot_bh_stride + s;
    float *img = p.S_slots + slot * S::DP * D;
#pragma unroll
    for (int f = 0; f < 2; f++)
#pragma unroll
        for (int vb = 0; vb < S::VB; vb++) {
            int e, hf, L;  // piece, half and lane of the reader that holds these four values
            if (D == 128) {
                // causal_ws_kernel_128: piece (4 fa + pv) 8 + j of lane (g, c), holding rows
                // 16 (8 fa + j) + 4 g + r, value columns value_col<2>(pv, h, c) in halves h.  Value
                // column 16 vb + r16 is in piece pv = vb / 2 at c = 4 (m / 8) + m % 4, half (m / 4) % 2,
                // with m = 16 (vb % 2) + r16; here fa = f, j = w.
                const int m = 16 * (vb & 1) + r16;
                e = (4 * f + (vb >> 1)) * 8 + w;
                L = 16 * g + 4 * (m >> 3) + (m & 3);
                hf = (m >> 2) & 1;
            } else {
                // wide_kernel<64>: piece wv 4 + j of lane (g, r16), wave wv owning value block wv,
                // holding rows 16 (2 j) + 4 g + r and 16 (2 j + 1) + 4 g + r of value column
                // 16 wv + r16 in its halves; here the feature block is 4 f + w.
                const int fb = 4 * f + w;
                e = vb * 4 + (fb >> 1);
                L = 16 * g + r16;
                hf = fb & 1;
            }
            *slot_piece(img, e, hf, L) = sacc[f][vb];
        }
    float *zs = p.z_slots + slot * S::DP;
    if (r16 == 0) {
#pragma unroll
        for (int f = 0; f < 2; f++)
#pragma unroll
            for (int r = 0; r < 4; r++) zs[16 * (S::NW * f + w) + 4 * g + r] = zacc[f][r];
    }
}

template <int D>
__global__ __launch_bounds__(StateSymCfg<D>::NT, StateSymCfg<D>::WG_PER_CU) void state_sym_kernel(WideParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[StateSymCfg<D>::LDS_BYTES];
    int bh, s;
    wg_head_segment(p.nseg_grid, bh, s);
    state_sym_body<D>(p, smem, bh, s);
}

// Bidirectional mode with one segment per sequence (d = 64): the total state S = phiK^T V,
// z = phiK^T 1 of the whole sequence and the read-out against it in one workgroup.  The state
// pass leaves the total in LDS, in the register image the read-out loads its slot from, instead
// of a workspace slot in memory that a second kernel reads back.
template <int D>
struct BidirFusedCfg {
    static constexpr int SLOT_S = 2 * D * D * 4;  // fp32 S image
    static constexpr int SLOT_Z = 2 * D * 4;      // fp32 z
    // The total lives after the read-out pass's tiles: the state pass writes it once its own tiles
    // are consumed, and the read-out's first loads (q staging, W) do not reach it before the
    // read-out has taken the total into registers.
    static constexpr int OFF_SLOT = (WideCfg<D, 64, WM_READOUT>::LDS_BYTES + 15) / 16 * 16;
    static constexpr int END_SLOT = OFF_SLOT + SLOT_S + SLOT_Z;
    static constexpr int TILES = StateSymCfg<D>::LDS_BYTES > END_SLOT ? StateSymCfg<D>::LDS_BYTES : END_SLOT;
    static_assert(StateSymCfg<D>::NT == WideCfg<D>::NT, "both passes use the same workgroup");
    static_assert(TILES * 2 <= 160 * 1024, "two workgroups per CU");
};

template <int D>
__global__ __launch_bounds__(WideCfg<D>::NT, 2) void bidir_fused_kernel(WideParams p) {
    using F = BidirFusedCfg<D>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[F::TILES];
    const int bh = blockIdx.x;
    WideParams q = p;
    q.S_slots = reinterpret_cast<float *>(smem + F::OFF_SLOT);  // generic pointers to LDS: slot 0 of every sequence
    q.z_slots = reinterpret_cast<float *>(smem + F::OFF_SLOT + F::SLOT_S);
    q.slot_bh_stride = 0;
    q.slot_mode = 2;
    state_sym_body<D>(q, smem, bh, 0);
    __syncthreads();  // the total is complete, the state pass's tiles are free
    wide_body<D, WM_READOUT>(q, smem, bh, 0);
}

hipError_t launch_bidir_fused(int d, const WideParams &p, int BH, hipStream_t st) {
    if (d != 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL(bidir_fused_kernel<64>, dim3(BH), dim3(WideCfg<64>::NT), 0, st, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Chunked causal pass for d = 128 with specialised waves (32-token chunks).
//   producers (waves 0-3, wave p): the scores of chunk c (query block x key block tasks),
//     then the feature maps of q and k of chunk c + 1, directions 32 p .. 32 p + 31;
//   consumers (waves 4-7, wave 4 + v): value columns 32 v .. 32 v + 31 of the state for all 256
//     features (no exchange between waves): read-out of chunk c and its normaliser partial
//     over features 64 v .. 64 v + 63, the state update with chunk c, and the finished output
//     of chunk c - 1 (intra-chunk product with the scores computed meanwhile).
// Each SIMD runs one producer and one consumer, one barrier per chunk.  Feature tiles,
// scores and normaliser slots are double-buffered, V triple-buffered (used by the update of
// chunk c and the intra product one chunk later), the raw q / k double-buffered and fetched
// two chunks ahead.
struct CausalWsCfg {
    static constexpr int D = 128, C = 32, DP = 256, NT = 512;
    // phi(q) [C][RQ] row-major (features in the permuted order); phi(k) transposed, [DP][PT]
    // (rows features in natural order, C tokens each, 96-byte rows), so that the consumers'
    // state-update operands (feature rows, K = tokens) are plain 16-byte reads
    static constexpr int RQ = DP + 16, PT = C + 16, RA = C + 8;
    static constexpr int SZ_PQ = C * RQ * 2, SZ_PK = DP * PT * 2, SZ_X = C * D * 2, SZ_A = C * RA * 2;
    // per token 8 floats: the 4 consumers' normaliser partials, the 2 score row sums, 2 unused
    // (one 16-byte and one 8-byte read give a token's six terms)
    static constexpr int NDEN = 8;
    static constexpr int SZ_DEN = NDEN * C * 4;
    static constexpr int OFF_PQ = 0;
    static constexpr int OFF_PK = OFF_PQ + 2 * SZ_PQ;
    static constexpr int OFF_V = OFF_PK + 2 * SZ_PK;
    static constexpr int OFF_A = OFF_V + 3 * SZ_X;
    static constexpr int OFF_DEN = OFF_A + 2 * SZ_A;
    static constexpr int OFF_XQ = OFF_DEN + 2 * SZ_DEN;
    static constexpr int OFF_XK = OFF_XQ + 2 * SZ_X;
    static constexpr int OFF_W = 0;
    static constexpr int OFF_SYNC = OFF_XK + 2 * SZ_X;   // producers' arrival counter
    // softmax maps: the two producer pairs' arrival counters, then the normaliser partials
    // [pair (token block)][direction half][q, k][max, sum][feature half][16 tokens]
    static constexpr int OFF_PAIR = OFF_SYNC + 16;
    static constexpr int OFF_PART = OFF_PAIR + 16;
    static constexpr int LDS_BYTES = OFF_PART + 2 * 2 * 2 * 2 * 2 * 16 * 4;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(D * D * 2 <= 2 * SZ_PQ + 2 * SZ_PK, "W fits in the feature tiles");
};

// Producer p: q and k features of token block p & 1 of a 32-token chunk, for directions
// 64 (p >> 1) .. 64 (p >> 1) + 63 (so each producer reads only its 16 tokens of q and k).  All
// operand reads first, then the eight independent product chains, then the exponentials, so
// that one wave keeps the LDS, matrix and vector pipes busy at once.
// Barrier of the four producer waves alone, on a counter in LDS (the consumers take no part: they
// are summing their starting state meanwhile).  Each producer's LDS writes and landed direct loads
// are complete before it arrives; `target` counts arrivals since the counter was cleared.
__device__ __forceinline__ void producer_barrier(unsigned int *cnt, unsigned int target, int lane) {
    __builtin_amdgcn_s_waitcnt(0);
    if (lane == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    while (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target) __builtin_amdgcn_s_sleep(1);
}

// Softmax maps (SM): the features of a token are exp(+-u - m) / sum over the half, u = W x without
// a bias.  Producer p holds 64 of the 128 directions of its 16 tokens; it forms the maximum m_p
// and the sum s_p of exp(x - m_p) over them, exchanges (m_p, s_p) with the producer holding the
// other 64 directions (p ^ 2, the same token block) through LDS, and scales its exponentials by
// exp(m_p - m) / (s_p exp(m_p - m) + s_q exp(m_q - m)), m = max(m_p, m_q).  `part` and `pcnt`
// are the partials and the pair's arrival counter; ncall counts this producer's calls.
// KO: the keys' features only (the segment-state mode of the chunked pass).
template <bool FULL, bool SM = false, bool KO = false>
__device__ __forceinline__ void cws_features(const unsigned char *xq, const unsigned char *xk, int valid,
                                             const bf16x8 (&wA)[4][4], const float (&bl2)[4][4],
                                             const float (&bk2)[4], int p, int g, int r16, bf16_t *sPQ,
                                             bf16_t *sPKT, float *part = nullptr, unsigned int *pcnt = nullptr,
                                             unsigned int *ncall = nullptr) {
    using S = CausalWsCfg;
    const int i = 16 * (p & 1) + r16;
    bf16x8 xb[2][4];  // [keys, queries][K step]
#pragma unroll
    for (int t = 0; t < (KO ? 1 : 2); t++)
#pragma unroll
        for (int ks = 0; ks < 4; ks++) xb[t][ks] = staged_x_operand<128>(t == 0 ? xk : xq, i, ks, g);
    // keys: u (tokens x directions), lane: direction 64 (p >> 1) + 16 mb + r16, tokens 4 g + r;
    // queries: u^T (directions x tokens), lane: token i, directions 64 (p >> 1) + 16 mb + 4 g + r.
    // The A and B operands hold the same per-lane data, so only their roles swap.
    f32x4 acc[2][4];
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
        for (int mb = 0; mb < 4; mb++) acc[t][mb] = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
            acc[0][mb] = mfma_bf16(xb[0][ks], wA[mb][ks], acc[0][mb]);
            if constexpr (!KO) acc[1][mb] = mfma_bf16(wA[mb][ks], xb[1][ks], acc[1][mb]);
        }
    const int f0 = 64 * (p >> 1) + 4 * g;
    if constexpr (SM) {
        // exponents in base 2; keys: lane direction 64 (p >> 1) + 16 mb + r16, token 4 g + r of the
        // block; queries: lane token r16, directions 64 (p >> 1) + 16 mb + 4 g + r
        f32x4 kp[4], kn[4], qp[4], qn[4];
        float km[2][4], ksum[2][4], qm[2], qsum[2];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            float a = -INFINITY, b = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 4; mb++) {
                const float x = acc[0][mb][r] * kLog2e;
                a = fmaxf(a, x);
                b = fmaxf(b, -x);
            }
            km[0][r] = row16_max(a);
            km[1][r] = row16_max(b);
        }
        if constexpr (!KO) {
            float a = -INFINITY, b = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 4; mb++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const float x = acc[1][mb][r] * kLog2e;
                    a = fmaxf(a, x);
                    b = fmaxf(b, -x);
                }
            a = fmaxf(a, __shfl_xor(a, 16));
            b = fmaxf(b, __shfl_xor(b, 16));
            qm[0] = fmaxf(a, __shfl_xor(a, 32));
            qm[1] = fmaxf(b, __shfl_xor(b, 32));
        }
#pragma unroll
        for (int r = 0; r < 4; r++) {
            float a = 0.0f, b = 0.0f;
#pragma unroll
            for (int mb = 0; mb < 4; mb++) {
                const float x = acc[0][mb][r] * kLog2e;
                kp[mb][r] = exp2_fast(x - km[0][r]);
                kn[mb][r] = exp2_fast(-x - km[1][r]);
                a += kp[mb][r];
                b += kn[mb][r];
            }
            ksum[0][r] = row16_sum(a);
            ksum[1][r] = row16_sum(b);
        }
        if constexpr (!KO) {
            float a = 0.0f, b = 0.0f;
#pragma unroll
            for (int mb = 0; mb < 4; mb++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const float x = acc[1][mb][r] * kLog2e;
                    qp[mb][r] = exp2_fast(x - qm[0]);
                    qn[mb][r] = exp2_fast(-x - qm[1]);
                    a += qp[mb][r];
                    b += qn[mb][r];
                }
            a += __shfl_xor(a, 16);
            b += __shfl_xor(b, 16);
            qsum[0] = a + __shfl_xor(a, 32);
            qsum[1] = b + __shfl_xor(b, 32);
        }
        // publish this producer's partials, meet the partner, combine
        auto slot = [&](int dh, int qk, int ms, int hf) { return part + ((((p & 1) * 2 + dh) * 2 + qk) * 2 + ms) * 32 + 16 * hf; };
        const int dh = p >> 1;
        if (r16 == 0) {
#pragma unroll
            for (int hf = 0; hf < 2; hf++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    slot(dh, 1, 0, hf)[4 * g + r] = km[hf][r];
                    slot(dh, 1, 1, hf)[4 * g + r] = ksum[hf][r];
                }
        }
        if (!KO && g == 0) {
#pragma unroll
            for (int hf = 0; hf < 2; hf++) {
                slot(dh, 0, 0, hf)[r16] = qm[hf];
                slot(dh, 0, 1, hf)[r16] = qsum[hf];
            }
        }
        *ncall += 1;
        producer_barrier(pcnt, 2u * *ncall, 16 * g + r16);
        float kc[2][4], qc[2];
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float mo = slot(dh ^ 1, 1, 0, hf)[4 * g + r], so = slot(dh ^ 1, 1, 1, hf)[4 * g + r];
                const float m = fmaxf(km[hf][r], mo);
                const float e = exp2_fast(km[hf][r] - m);
                kc[hf][r] = e * __builtin_amdgcn_rcpf(fmaf(ksum[hf][r], e, so * exp2_fast(mo - m)));
            }
            if constexpr (!KO) {
                const float mo = slot(dh ^ 1, 0, 0, hf)[r16], so = slot(dh ^ 1, 0, 1, hf)[r16];
                const float m = fmaxf(qm[hf], mo);
                const float e = exp2_fast(qm[hf] - m);
                qc[hf] = e * __builtin_amdgcn_rcpf(fmaf(qsum[hf], e, so * exp2_fast(mo - m)));
            }
        }
        const int fk = 64 * (p >> 1) + r16;
        const int tk = 16 * (p & 1) + 4 * g;
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
            f32x4 ep, en;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                ep[r] = kp[mb][r] * kc[0][r];
                en[r] = kn[mb][r] * kc[1][r];
                if (!FULL && tk + r >= valid) ep[r] = en[r] = 0.0f;  // keys past the end contribute nothing
            }
            store4(sPKT + (fk + 16 * mb) * S::PT + tk, to_bf16x4(ep));
            store4(sPKT + (128 + fk + 16 * mb) * S::PT + tk, to_bf16x4(en));
        }
        if constexpr (KO) return;
        bf16x4 pe[4], ne[4];
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
            f32x4 ep, en;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                ep[r] = qp[mb][r] * qc[0];
                en[r] = qn[mb][r] * qc[1];
            }
            pe[mb] = to_bf16x4(ep);
            ne[mb] = to_bf16x4(en);
        }
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
            store8(sPQ + i * S::RQ + feat_pos<true>(f0 + 32 * hh), cat(pe[2 * hh], pe[2 * hh + 1]));
            store8(sPQ + i * S::RQ + feat_pos<true>(128 + f0 + 32 * hh), cat(ne[2 * hh], ne[2 * hh + 1]));
        }
        return;
    }
    {  // keys: phi(k)^T rows 64 (p >> 1) + 16 mb + r16 and 128 + that, tokens 16 (p & 1) + 4 g .. + 3
        const int fk = 64 * (p >> 1) + r16;
        const int tk = 16 * (p & 1) + 4 * g;
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
            f32x4 ep, en;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float u = acc[0][mb][r] * kLog2e + bk2[mb];
                ep[r] = exp2_fast(u);
                en[r] = exp2_fast(-u);
                if (!FULL && tk + r >= valid) ep[r] = en[r] = 0.0f;  // keys past the end contribute nothing
            }
            store4(sPKT + (fk + 16 * mb) * S::PT + tk, to_bf16x4(ep));
            store4(sPKT + (128 + fk + 16 * mb) * S::PT + tk, to_bf16x4(en));
        }
    }
    if constexpr (!KO) {  // queries: direction blocks 2 h, 2 h + 1 share one 16-byte run of their 32-feature group
        bf16x4 pe[4], ne[4];
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
            f32x4 ep, en;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float u = acc[1][mb][r] * kLog2e + bl2[mb][r];
                ep[r] = exp2_fast(u);
                en[r] = exp2_fast(-u);
            }
            pe[mb] = to_bf16x4(ep);
            ne[mb] = to_bf16x4(en);
        }
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
            store8(sPQ + i * S::RQ + feat_pos<true>(f0 + 32 * hh), cat(pe[2 * hh], pe[2 * hh + 1]));
            store8(sPQ + i * S::RQ + feat_pos<true>(128 + f0 + 32 * hh), cat(ne[2 * hh], ne[2 * hh + 1]));
        }
    }
}

// Full chunks skip the per-lane masking of keys past the end.
template <bool SM = false, bool KO = false>
__device__ __forceinline__ void cws_features_any(const unsigned char *xq, const unsigned char *xk, int valid,
                                                 const bf16x8 (&wA)[4][4], const float (&bl2)[4][4],
                                                 const float (&bk2)[4], int p, int g, int r16, bf16_t *sPQ,
                                                 bf16_t *sPKT, float *part = nullptr, unsigned int *pcnt = nullptr,
                                                 unsigned int *ncall = nullptr) {
    if (valid >= CausalWsCfg::C)
        cws_features<true, SM, KO>(xq, xk, valid, wA, bl2, bk2, p, g, r16, sPQ, sPKT, part, pcnt, ncall);
    else
        cws_features<false, SM, KO>(xq, xk, valid, wA, bl2, bk2, p, g, r16, sPQ, sPKT, part, pcnt, ncall);
}

// MFMA operand from the transposed phi(k) tile in the permuted feature order of phi(q): lane
// (g, r16) gets key c0 + r16 and features r0 + 4 g .. + 3, r0 + 16 + 4 g .. + 3 (two transposing
// reads; lane_off_p = (4 g + r16 / 4) PT + 4 (r16 % 4)).
__device__ __forceinline__ bf16x8 pkt_operand_perm(const bf16_t *sPKT, int lane_off_p, int r0, int c0) {
    const bf16_t *p = sPKT + lane_off_p + r0 * CausalWsCfg::PT + c0;
    return cat(lds_read_tr(p), lds_read_tr(p + 16 * CausalWsCfg::PT));
}

// Producer: scores of one chunk.  Tasks: p0 (0,0), p1 (1,0), p2 (1,1); p3 clears the masked
// block (0,1) and the second row-sum slot of query block 0.
__device__ __forceinline__ void cws_scores(const bf16_t *sPQ, const bf16_t *sPKT, bf16_t *sA, float *sDen, int p,
                                           int g, int r16) {
    using S = CausalWsCfg;
    if (p == 3) {
        bf16x4 zz;
        zz[0] = zz[1] = zz[2] = zz[3] = (__bf16)0.0f;
        store4(sA + r16 * S::RA + 16 + 4 * g, zz);
        sDen[r16 * S::NDEN + 5] = 0.0f;
        return;
    }
    const int ib = p == 0 ? 0 : 1, jb = p == 2 ? 1 : 0, slot = p == 2 ? 5 : 4;
    // all operand reads first, then two product chains over alternate K steps
    bf16x8 ka[8], qb[8];
    const int lop = (4 * g + (r16 >> 2)) * S::PT + 4 * (r16 & 3);
#pragma unroll
    for (int ks = 0; ks < 8; ks++) {
        ka[ks] = pkt_operand_perm(sPKT, lop, 32 * ks, 16 * jb);
        qb[ks] = load8(sPQ + (16 * ib + r16) * S::RQ + 32 * ks + 8 * g);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 a2[2] = {zero4(), zero4()};
#pragma unroll
    for (int ks = 0; ks < 8; ks++) a2[ks & 1] = mfma_bf16(ka[ks], qb[ks], a2[ks & 1]);
    f32x4 a = a2[0] + a2[1];
    // a = A^T[j][i]: lane holds i = 16 ib + r16, j = 16 jb + 4 g + r; keep j <= i
    if (jb == ib) {
#pragma unroll
        for (int r = 0; r < 4; r++)
            if (4 * g + r > r16) a[r] = 0.0f;
    }
    const bf16x4 ab = to_bf16x4(a);
    float rs = ((float)ab[0] + (float)ab[1]) + ((float)ab[2] + (float)ab[3]);
    store4(sA + (16 * ib + r16) * S::RA + 16 * jb + 4 * g, ab);
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    sDen[(16 * ib + r16) * S::NDEN + slot] = rs;  // the same value in all four lane groups
}

// Normaliser of token i: the sum of its six partial terms.
__device__ __forceinline__ float den_terms(const float *sDen, int i) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(sDen + i * CausalWsCfg::NDEN);
    const float2 b = *reinterpret_cast<const float2 *>(sDen + i * CausalWsCfg::NDEN + 4);
    return ((a[0] + a[1]) + (a[2] + a[3])) + (b.x + b.y);
}

// Consumer: finish the outputs of one chunk (held read-out + intra-chunk product, normalise,
// store).  Lane (g, r16) owns token 16 ib + r16, value columns value_col<2>(v, vb, 4 g + r).
__device__ __forceinline__ void cws_output(f32x4 (&numT)[2][2], const bf16_t *sA, const bf16_t *sV, const float *sDen,
                                           int lane_v, bf16_t *__restrict__ yrow0, int valid, int v, int g, int r16) {
    using S = CausalWsCfg;
    bf16x8 vop[2];
#pragma unroll
    for (int vb = 0; vb < 2; vb++) vop[vb] = operand_down_rows(sV, lane_v, 4 * vb, S::D);
#pragma unroll
    for (int ib = 0; ib < 2; ib++) {
        const int i = 16 * ib + r16;
        const bf16x8 a = load8(sA + i * S::RA + 8 * g);
#pragma unroll
        for (int vb = 0; vb < 2; vb++) numT[ib][vb] = mfma_bf16(vop[vb], a, numT[ib][vb]);
        const float rden = __builtin_amdgcn_rcpf(den_terms(sDen, i));
        f32x4 o0, o1;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            o0[r] = numT[ib][0][r] * rden;
            o1[r] = numT[ib][1][r] * rden;
        }
        if (i < valid) store8(yrow0 + (size_t)i * S::D + value_col<2>(v, 0, 4 * g), cat(to_bf16x4(o0), to_bf16x4(o1)));
    }
}

// Inputs of chunk c + 1 (V) and c + 2 (q, k) into the buffers freed by the last chunk; issued by
// every wave (each moves its own 1 KB blocks).
// ST: no query tiles (the segment-state mode).
template <bool ST = false>
__device__ __forceinline__ void cws_issue(const WideParams &p, const DmaLanes128<32> &dl, size_t base, int t_begin,
                                          int t_end, int c, int n, int w, unsigned char *smem) {
    using S = CausalWsCfg;
    if (c + 1 < n) {
        const int t = t_begin + S::C * (c + 1);
        dl.issue<true>(p.v + base, t, min(S::C, t_end - t), w, smem + S::OFF_V + ((c + 1) % 3) * S::SZ_X);
    }
    if (c + 2 < n) {
        const int t = t_begin + S::C * (c + 2), b = c & 1;
        if (!ST) dl.issue<false>(p.q + base, t, min(S::C, t_end - t), w, smem + S::OFF_XQ + b * S::SZ_X);
        dl.issue<false>(p.k + base, t, min(S::C, t_end - t), w, smem + S::OFF_XK + b * S::SZ_X);
    }
}


// SM: the per-half softmax map (no bias; see cws_features) instead of the Hedgehog map.
// ST: segment-state mode: the same pipeline with the keys' features only and the consumers'
// state update alone, from a zero state; the segment's aggregate is written to its slot.
template <bool SM = false, bool ST = false>
__global__ __launch_bounds__(512, 1) void causal_ws_kernel_128(WideParams p) {
    using S = CausalWsCfg;
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::LDS_BYTES];
    const int tid = threadIdx.x;
    // wave index as a scalar: role branches on it stay scalar (never exec-masked around MFMAs)
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int pv = w & 3;  // producer index / consumer value part
    int bh, s;
    wg_head_segment(p.nseg_grid, bh, s);
    const int h = bh % p.H;
    const int t_begin = s * p.seg_len;
    const int t_end = min(p.N, t_begin + p.seg_len);
    const size_t base = (size_t)bh * p.N * S::D;
    const int n = t_end > t_begin ? (t_end - t_begin + S::C - 1) / S::C : 0;
    const DmaLanes128<32> dl(w, lane);
    auto valid_of = [&](int c) { return min(S::C, t_end - (t_begin + S::C * c)); };
    auto pq_buf = [&](int b) { return reinterpret_cast<bf16_t *>(smem + S::OFF_PQ + b * S::SZ_PQ); };
    auto pk_buf = [&](int b) { return reinterpret_cast<bf16_t *>(smem + S::OFF_PK + b * S::SZ_PK); };  // phi(k)^T
    auto v_buf = [&](int b) { return reinterpret_cast<const bf16_t *>(smem + S::OFF_V + b * S::SZ_X); };
    auto a_buf = [&](int b) { return reinterpret_cast<bf16_t *>(smem + S::OFF_A + b * S::SZ_A); };
    auto den_buf = [&](int b) { return reinterpret_cast<float *>(smem + S::OFF_DEN + b * S::SZ_DEN); };

    unsigned int *psync = reinterpret_cast<unsigned int *>(smem + S::OFF_SYNC);
    unsigned int *ppair = reinterpret_cast<unsigned int *>(smem + S::OFF_PAIR);  // [token block]
    float *part = reinterpret_cast<float *>(smem + S::OFF_PART);
    if (tid == 0) {
        *psync = 0u;
        ppair[0] = ppair[1] = 0u;
    }
    __syncthreads();
    // The two roles run separate streams with the same barriers: one before the first chunk, then
    // one per chunk.
    if (w < 4) {
        unsigned int ncall = 0;  // feature-map calls of this producer (softmax maps: pair meetings)
        bf16x8 wA[4][4];  // W operands, directions 64 (pv >> 1) .. + 63
        float bl2[4][4];  // bias x log2(e) of the query accumulators' rows (directions 16 mb + 4 g + r)
        float bk2[4];     // and of the key accumulators' column (direction 16 mb + r16)
        // Producers issue every staging load of the prologue (each moves the 1 KB blocks of waves w
        // and w + 4 of the eight-wave layout), so that the consumers' load queues hold only their
        // own prefix loads below: loads retire in order per wave, and a consumer waiting for a prefix
        // slot then never waits for staging traffic as well.
#pragma unroll
        for (int hw = 0; hw < 2; hw++) {
            const int vw = w + 4 * hw;
            if (n > 0) {
                if (!ST) stage_x<128, 32>(p.q + base, t_begin, valid_of(0), vw, lane, smem + S::OFF_XQ);
                stage_x<128, 32>(p.k + base, t_begin, valid_of(0), vw, lane, smem + S::OFF_XK);
                stage_v<128, 32>(p.v + base, t_begin, valid_of(0), vw, lane, smem + S::OFF_V);
            }
            if (n > 1) {
                if (!ST)
                    stage_x<128, 32>(p.q + base, t_begin + S::C, valid_of(1), vw, lane, smem + S::OFF_XQ + S::SZ_X);
                stage_x<128, 32>(p.k + base, t_begin + S::C, valid_of(1), vw, lane, smem + S::OFF_XK + S::SZ_X);
            }
            stage_w_dma128(p.W, h, vw, lane, smem + S::OFF_W);
        }
        // Then, while the consumers sum their starting state, the W operands and the feature maps of
        // the first chunk (W shares space with the feature tiles: every producer has read it before
        // any feature is written).
        producer_barrier(psync, 4, lane);
        // the two 32-direction groups 2 (pv >> 1), 2 (pv >> 1) + 1
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
            bf16x8 w2[2][4];
            float b2[2][4];
            load_w_operands<128>(smem + S::OFF_W, 2 * (pv >> 1) + hh, g, r16, w2);
            load_bias<128>(p.b, h, 2 * (pv >> 1) + hh, g, b2);
#pragma unroll
            for (int mb = 0; mb < 2; mb++) {
#pragma unroll
                for (int ks = 0; ks < 4; ks++) wA[2 * hh + mb][ks] = w2[mb][ks];
#pragma unroll
                for (int r = 0; r < 4; r++) bl2[2 * hh + mb][r] = b2[mb][r];
            }
        }
#pragma unroll
        for (int mb = 0; mb < 4; mb++) bk2[mb] = 0.0f;
        if (p.b) {
#pragma unroll
            for (int mb = 0; mb < 4; mb++)
                bk2[mb] = bf16_bits_to_float(p.b[(size_t)h * 128 + 64 * (pv >> 1) + 16 * mb + r16]) * kLog2e;
        }
        producer_barrier(psync, 8, lane);
        if (n > 0)
            cws_features_any<SM, ST>(smem + S::OFF_XQ, smem + S::OFF_XK, valid_of(0), wA, bl2, bk2, pv, g, r16,
                                     pq_buf(0), pk_buf(0), part, ppair + (pv & 1), &ncall);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int c = 0; c < n; c++) {
            cws_issue<ST>(p, dl, base, t_begin, t_end, c, n, w, smem);
            const int b2 = c & 1;
            if (!ST) cws_scores(pq_buf(b2), pk_buf(b2), a_buf(b2), den_buf(b2), pv, g, r16);
            if (c + 1 < n)
                cws_features_any<SM, ST>(smem + S::OFF_XQ + (b2 ^ 1) * S::SZ_X,
                                         smem + S::OFF_XK + (b2 ^ 1) * S::SZ_X, valid_of(c + 1), wA, bl2, bk2, pv, g,
                                         r16, pq_buf(b2 ^ 1), pk_buf(b2 ^ 1), part, ppair + (pv & 1), &ncall);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        return;
    }
    // Consumer state: value columns value_col<2>(pv, vb, c) of S for all 256 features, z rows of
    // feature blocks 4 pv .. 4 pv + 3.
    f32x4 sacc[16][2];
    f32x4 zacc[4];
    {
        // Starting state: the caller's S0, plus the earlier segments' contribution.  slot_mode 1:
        // slot s holds their exclusive prefix; slot_mode 3: slots 0 .. s - 1 hold their aggregates
        // (written by the segment-state pass just before, by workgroups of the same XCD), summed
        // here in fp32 while the producers' staging loads are in flight.
#pragma unroll
        for (int fb = 0; fb < 16; fb++) sacc[fb][0] = sacc[fb][1] = zero4();
#pragma unroll
        for (int zb = 0; zb < 4; zb++) zacc[zb] = zero4();
        if (!ST && p.S_in) {
            const float *Si = p.S_in + (size_t)bh * p.in_bh_stride * S::DP * S::D;
            const float *zi = p.z_in + (size_t)bh * p.in_bh_stride * S::DP;
#pragma unroll
            for (int fb = 0; fb < 16; fb++)
#pragma unroll
                for (int vb = 0; vb < 2; vb++) {
                    const int nn = value_col<2>(pv, vb, r16);
#pragma unroll
                    for (int r = 0; r < 4; r++) sacc[fb][vb][r] = Si[(size_t)(16 * fb + 4 * g + r) * S::D + nn];
                }
#pragma unroll
            for (int zb = 0; zb < 4; zb++)
#pragma unroll
                for (int r = 0; r < 4; r++) zacc[zb][r] = zi[16 * (4 * pv + zb) + 4 * g + r];
        }
        int t0 = 0, t1 = 0;  // slots to add
        if (!ST && s > 0 && p.slot_mode == 1) t0 = s, t1 = s + 1;
        if (!ST && s > 0 && p.slot_mode == 3) t0 = 0, t1 = s;
        for (int t = t0; t < t1; t++) {
            const size_t sl = (size_t)bh * p.slot_bh_stride + t;
            const float *zs = p.z_slots + sl * S::DP;
            const float *img = p.S_slots + sl * S::DP * S::D;
            f32x4 zslot[4];
#pragma unroll
            for (int zb = 0; zb < 4; zb++) zslot[zb] = *reinterpret_cast<const f32x4 *>(zs + 16 * (4 * pv + zb) + 4 * g);
            // the slot in two halves of 64 registers (the state itself holds 128)
#pragma unroll
            for (int fa = 0; fa < 2; fa++) {
                f32x4 slot_raw[8][2];
#pragma unroll
                for (int j = 0; j < 8; j++)
#pragma unroll
                    for (int hf = 0; hf < 2; hf++) slot_raw[j][hf] = *slot_piece(img, (4 * fa + pv) * 8 + j, hf, lane);
                __builtin_amdgcn_sched_barrier(0);  // the half's loads in flight before its first sum
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    sacc[8 * fa + j][0] += slot_raw[j][0];
                    sacc[8 * fa + j][1] += slot_raw[j][1];
                }
            }
#pragma unroll
            for (int zb = 0; zb < 4; zb++)
#pragma unroll
                for (int r = 0; r < 4; r++) zacc[zb][r] += zslot[zb][r];
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const int r0 = 8 * g + (r16 >> 2);
    const int lane_v = r0 * S::D + 8 * v_pos(r0, 4 * pv + (r16 & 3));
    const bf16x8 ones = ones_bf16x8();
    if constexpr (ST) {
        // the update alone: S += phi(K)^T V and z += phi(K)^T 1 per chunk, as in the loop below
        for (int c = 0; c < n; c++) {
            cws_issue<true>(p, dl, base, t_begin, t_end, c, n, w, smem);
            const bf16_t *sPK = pk_buf(c & 1);
            const bf16_t *sV = v_buf(c % 3);
            bf16x8 vop[2], an[2];
#pragma unroll
            for (int vb = 0; vb < 2; vb++) vop[vb] = operand_down_rows(sV, lane_v, 4 * vb, S::D);
#pragma unroll
            for (int j = 0; j < 2; j++) an[j] = load8(sPK + (16 * j + r16) * S::PT + 8 * g);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < 8; ks++) {
                const bf16x8 ac[2] = {an[0], an[1]};
                if (ks < 7) {
#pragma unroll
                    for (int j = 0; j < 2; j++) an[j] = load8(sPK + (32 * (ks + 1) + 16 * j + r16) * S::PT + 8 * g);
                }
#pragma unroll
                for (int j = 0; j < 2; j++)
#pragma unroll
                    for (int vb = 0; vb < 2; vb++)
                        sacc[2 * ks + j][vb] = mfma_bf16(ac[j], vop[vb], sacc[2 * ks + j][vb]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int zb = 0; zb < 4; zb++)
                zacc[zb] = mfma_bf16(load8(sPK + (16 * (4 * pv + zb) + r16) * S::PT + 8 * g), ones, zacc[zb]);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        // slot s: each accumulator as the 16-byte piece the slot sum above reads it back from
        const size_t sl = (size_t)bh * p.slot_bh_stride + s;
        float *img = p.S_slots + sl * S::DP * S::D;
#pragma unroll
        for (int fa = 0; fa < 2; fa++)
#pragma unroll
            for (int j = 0; j < 8; j++)
#pragma unroll
                for (int vb = 0; vb < 2; vb++) *slot_piece(img, (4 * fa + pv) * 8 + j, vb, lane) = sacc[8 * fa + j][vb];
        if (r16 == 0) {
            float *zs = p.z_slots + sl * S::DP;
#pragma unroll
            for (int zb = 0; zb < 4; zb++)
#pragma unroll
                for (int r = 0; r < 4; r++) zs[16 * (4 * pv + zb) + 4 * g + r] = zacc[zb][r];
        }
        return;
    }

    f32x4 numT[2][2];
#pragma unroll
    for (int ib = 0; ib < 2; ib++) numT[ib][0] = numT[ib][1] = zero4();
    bf16_t *ybase = p.y + base;

    for (int c = 0; c < n; c++) {
        cws_issue(p, dl, base, t_begin, t_end, c, n, w, smem);
        const int b2 = c & 1;
        const bf16_t *sPQ = pq_buf(b2);
        const bf16_t *sPK = pk_buf(b2);
        // One branch-free stream per chunk: the outputs of chunk c - 1 (intra-chunk product with
        // its scores, normalisation, store) ride along the first K steps of the read-out of chunk
        // c (transposed, into nt) and the state update with chunk c.  The state update of K step
        // ks (feature blocks 2 ks, 2 ks + 1) follows that step's read-out, which has already taken
        // the state's bf16 operand.  Operands of K step ks + 1 are read while the products of
        // step ks run; the scheduling fences keep the reads ahead of the products.
        const bf16_t *sVp = v_buf((c + 2) % 3);
        const bf16_t *sAp = a_buf(b2 ^ 1);
        const float *sDp = den_buf(b2 ^ 1);
        bf16x8 vp[2], ao[2];
#pragma unroll
        for (int vb = 0; vb < 2; vb++) vp[vb] = operand_down_rows(sVp, lane_v, 4 * vb, S::D);
#pragma unroll
        for (int ib = 0; ib < 2; ib++) ao[ib] = load8(sAp + (16 * ib + r16) * S::RA + 8 * g);
        const bf16_t *sV = v_buf(c % 3);
        bf16x8 vop[2];
#pragma unroll
        for (int vb = 0; vb < 2; vb++) vop[vb] = operand_down_rows(sV, lane_v, 4 * vb, S::D);
        bf16x8 qn[2], an[2];
        auto load_step = [&](int ks, bf16x8(&qo)[2], bf16x8(&ao2)[2]) {
#pragma unroll
            for (int ib = 0; ib < 2; ib++) qo[ib] = load8(sPQ + (16 * ib + r16) * S::RQ + 32 * ks + 8 * g);
#pragma unroll
            for (int j = 0; j < 2; j++) ao2[j] = load8(sPK + (32 * ks + 16 * j + r16) * S::PT + 8 * g);
        };
        load_step(0, qn, an);
        // the read-out and update products at raised wave priority: when both waves of a SIMD
        // have an instruction ready, the consumer's products go first (the producer's vector
        // work fills the matrix pipe's busy cycles)
        __builtin_amdgcn_s_setprio(2);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 nt[2][2];
#pragma unroll
        for (int ib = 0; ib < 2; ib++) nt[ib][0] = nt[ib][1] = zero4();
        float dsum[2];
#pragma unroll
        for (int ks = 0; ks < 8; ks++) {
            bf16x8 qc[2] = {qn[0], qn[1]}, ac[2] = {an[0], an[1]};
            if (ks < 7) load_step(ks + 1, qn, an);
            if (ks == 0) {  // intra-chunk product of chunk c - 1
#pragma unroll
                for (int ib = 0; ib < 2; ib++)
#pragma unroll
                    for (int vb = 0; vb < 2; vb++) numT[ib][vb] = mfma_bf16(vp[vb], ao[ib], numT[ib][vb]);
            }
            if (ks == 1) {  // its normaliser: the partial terms of every wave
#pragma unroll
                for (int ib = 0; ib < 2; ib++) dsum[ib] = den_terms(sDp, 16 * ib + r16);
            }
            bf16x8 sb[2];
#pragma unroll
            for (int vb = 0; vb < 2; vb++) sb[vb] = acc_pair_to_operand(sacc[2 * ks][vb], sacc[2 * ks + 1][vb]);
#pragma unroll
            for (int ib = 0; ib < 2; ib++)
#pragma unroll
                for (int vb = 0; vb < 2; vb++) nt[ib][vb] = mfma_bf16(sb[vb], qc[ib], nt[ib][vb]);
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int vb = 0; vb < 2; vb++) sacc[2 * ks + j][vb] = mfma_bf16(ac[j], vop[vb], sacc[2 * ks + j][vb]);
            if (ks == 2 && c > 0) {  // outputs of chunk c - 1 (every token of it is valid)
                bf16_t *yrow0 = ybase + (size_t)(t_begin + S::C * (c - 1)) * S::D;
#pragma unroll
                for (int ib = 0; ib < 2; ib++) {
                    const float rden = __builtin_amdgcn_rcpf(dsum[ib]);
                    f32x4 o0, o1;
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        o0[r] = numT[ib][0][r] * rden;
                        o1[r] = numT[ib][1][r] * rden;
                    }
                    store8(yrow0 + (size_t)(16 * ib + r16) * S::D + value_col<2>(pv, 0, 4 * g),
                           cat(to_bf16x4(o0), to_bf16x4(o1)));
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int ib = 0; ib < 2; ib++) {
            numT[ib][0] = nt[ib][0];
            numT[ib][1] = nt[ib][1];
        }
        __builtin_amdgcn_s_setprio(0);
        f32x4 dacc[2] = {zero4(), zero4()};
        {
            const bf16_t *sPQz = sPQ + 64 * pv;  // K steps 2 pv, 2 pv + 1
#pragma unroll
            for (int kz = 0; kz < 2; kz++) {
                const bf16x8 zop = acc_pair_to_operand(zacc[2 * kz], zacc[2 * kz + 1]);
#pragma unroll
                for (int ib = 0; ib < 2; ib++)
                    dacc[ib] = mfma_bf16(zop, load8(sPQz + (16 * ib + r16) * S::RQ + 32 * kz + 8 * g), dacc[ib]);
            }
        }
        // every row of dacc holds the token's partial: all four lane groups write the same value
        float *sDen = den_buf(b2);
        sDen[r16 * S::NDEN + pv] = dacc[0][0];
        sDen[(16 + r16) * S::NDEN + pv] = dacc[1][0];
        {  // normaliser rows of this consumer (feature blocks 4 pv .. 4 pv + 3)
#pragma unroll
            for (int zb = 0; zb < 4; zb++)
                zacc[zb] = mfma_bf16(load8(sPK + (16 * (4 * pv + zb) + r16) * S::PT + 8 * g), ones, zacc[zb]);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    if (n > 0) {
        cws_output(numT, a_buf((n - 1) & 1), v_buf((n - 1) % 3), den_buf((n - 1) & 1), lane_v,
                   ybase + (size_t)(t_begin + S::C * (n - 1)) * S::D, valid_of(n - 1), pv, g, r16);
    }
    if (p.S_out && s == p.nseg_grid - 1) {
        float *So = p.S_out + (size_t)bh * S::DP * S::D;
        float *zo = p.z_out + (size_t)bh * S::DP;
#pragma unroll
        for (int fb = 0; fb < 16; fb++)
#pragma unroll
            for (int vb = 0; vb < 2; vb++) {
                const int nn = value_col<2>(pv, vb, r16);
#pragma unroll
                for (int r = 0; r < 4; r++) So[(size_t)(16 * fb + 4 * g + r) * S::D + nn] = sacc[fb][vb][r];
            }
        if (r16 == 0) {
#pragma unroll
            for (int zb = 0; zb < 4; zb++)
#pragma unroll
                for (int r = 0; r < 4; r++) zo[16 * (4 * pv + zb) + 4 * g + r] = zacc[zb][r];
        }
    }
}

// ---------------------------------------------------------------------------------------
// Chunked causal pass for d = 64 with specialised waves: the d = 128 design at a quarter of
// its width.  One workgroup of eight waves runs two independent pipelines, the same segment of
// two sequences 2 j and 2 j + 1 (equal lengths, so both take the same barriers); pipeline q
// has producers on waves 2 q, 2 q + 1 and consumers on waves 4 + 2 q, 4 + 2 q + 1, so every
// SIMD (waves w and w + 4) pairs a producer with a consumer.  Per pipeline and 32-token chunk:
//   producer p (token block p): the q and k features of its 16 tokens for all 64 directions,
//     phi(q) row-major in the permuted feature order, phi(k) transposed (feature rows, natural
//     order); scores p0: blocks (0,0), (1,1); p1: block (1,0) and the masked block (0,1);
//   consumer v: value columns 32 v .. 32 v + 31 of the state for all 128 features and z of
//     feature blocks 4 v .. 4 v + 3: read-out, update, normaliser partial, and the outputs of
//     the chunk before (intra-chunk product with its scores).
// Segment slots are those of the d = 64 segment-state pass (the register image of the generic
// chunked kernel); a consumer reads each of its accumulators from there as one 16-byte piece.
struct CausalWs64Cfg {
    static constexpr int D = 64, C = 32, DP = 128, NT = 512;
    static constexpr int RQ = DP + 16, PT = C + 16, RA = C + 8;
    static constexpr int SZ_PQ = C * RQ * 2, SZ_PK = DP * PT * 2, SZ_X = C * D * 2, SZ_A = C * RA * 2;
    static constexpr int NDEN = 4;  // per token: the 2 consumers' normaliser partials, 2 score row sums
    static constexpr int SZ_DEN = NDEN * C * 4;
    static constexpr int OFF_PQ = 0;
    static constexpr int OFF_PK = OFF_PQ + 2 * SZ_PQ;
    static constexpr int OFF_V = OFF_PK + 2 * SZ_PK;
    static constexpr int OFF_A = OFF_V + 3 * SZ_X;
    static constexpr int OFF_DEN = OFF_A + 2 * SZ_A;
    static constexpr int OFF_XQ = OFF_DEN + 2 * SZ_DEN;
    static constexpr int OFF_XK = OFF_XQ + 2 * SZ_X;
    static constexpr int OFF_SYNC = OFF_XK + 2 * SZ_X;  // the producers' arrival counter
    static constexpr int PIPE_BYTES = OFF_SYNC + 16;
    static constexpr int LDS_BYTES = 2 * PIPE_BYTES;
    static_assert(PIPE_BYTES % 16 == 0, "pipelines 16-byte aligned");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Stored position of granule G (8 values) of row r in this kernel's V tiles (128-byte rows
// filled by direct loads): rotated by 4 on rows 2, 3 (mod 4), so the transposing reads of 16
// rows x 4 granules spread over both halves of the banks; the rotation repeats every 4 rows.
__device__ __forceinline__ int v_pos64(int r, int G) { return (G + 4 * ((r >> 1) & 1)) & 7; }

// Per-lane offsets of the direct loads of [32][64] bf16 tiles by the four waves of a pipeline
// (pipeline wave pw moves 1 KB block pw): byte offsets in the q / k staging layout (stage_pos)
// and in the V layout (v_pos64), and the row.  A row past the end reads the same granule of
// row 0 (x0, v0), a copy of row 0 in the tile's layout.
struct Dma64Lanes {
    uint32_t ox, ov, x0, v0;
    int row;
    __device__ __forceinline__ Dma64Lanes(int pw, int lane) {
        const int slot = 64 * pw + lane;
        const int r = slot / 8, P = slot % 8;
        row = r;
        const int gx = stage_granule<64>(r, P), gv = (P - 4 * ((r >> 1) & 1)) & 7;
        ox = 2 * (r * 64 + 8 * gx);
        ov = 2 * (r * 64 + 8 * gv);
        x0 = 16 * gx;
        v0 = 16 * gv;
    }
    template <bool V>
    __device__ __forceinline__ void issue(const bf16_t *x, int t0, int valid, int pw, unsigned char *stage) const {
        load_to_lds_16s(x + (size_t)t0 * 64, row < valid ? (V ? ov : ox) : (V ? v0 : x0), stage + 1024 * pw);
    }
};

// Producer p: features of token block p of a chunk for all 64 directions.
// SM: the per-half softmax map (no bias): a producer holds all 64 directions of its 16 tokens, so
// each token's maximum and sum are reduced inside the wave (keys over the 16 lanes of a group,
// queries over the four lane groups) and the features are stored normalised.
// KO: the keys' features only (the segment-state mode of the chunked pass).
template <bool FULL, bool SM = false, bool KO = false>
__device__ __forceinline__ void cw64_features(const unsigned char *xq, const unsigned char *xk, int valid,
                                              const bf16x8 (&wA)[4][2], const float (&bl2)[4][4],
                                              const float (&bk2)[4], int p, int g, int r16, bf16_t *sPQ,
                                              bf16_t *sPKT) {
    using S = CausalWs64Cfg;
    const int i = 16 * p + r16;
    bf16x8 xb[2][2];  // [keys, queries][K step]
#pragma unroll
    for (int t = 0; t < (KO ? 1 : 2); t++)
#pragma unroll
        for (int ks = 0; ks < 2; ks++) xb[t][ks] = staged_x_operand<64>(t == 0 ? xk : xq, i, ks, g);
    // keys: u (tokens x directions), lane: direction 16 mb + r16, tokens 16 p + 4 g + r;
    // queries: u^T (directions x tokens), lane: token i, directions 16 mb + 4 g + r
    f32x4 acc[2][4];
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
        for (int mb = 0; mb < 4; mb++) acc[t][mb] = zero4();
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
            acc[0][mb] = mfma_bf16(xb[0][ks], wA[mb][ks], acc[0][mb]);
            if constexpr (!KO) acc[1][mb] = mfma_bf16(wA[mb][ks], xb[1][ks], acc[1][mb]);
        }
    if constexpr (SM) {
        const int tk = 16 * p + 4 * g;
        // keys: lane direction 16 mb + r16, token 4 g + r of the block
        f32x4 kp[4], kn[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            float a = -INFINITY, b = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 4; mb++) {
                const float x = acc[0][mb][r] * kLog2e;
                a = fmaxf(a, x);
                b = fmaxf(b, -x);
            }
            const float mp = row16_max(a), mn = row16_max(b);
            float sp = 0.0f, sn = 0.0f;
#pragma unroll
            for (int mb = 0; mb < 4; mb++) {
                const float x = acc[0][mb][r] * kLog2e;
                kp[mb][r] = exp2_fast(x - mp);
                kn[mb][r] = exp2_fast(-x - mn);
                sp += kp[mb][r];
                sn += kn[mb][r];
            }
            const float zp = row16_sum(sp), zn = row16_sum(sn);  // (every lane takes part)
            const bool live = FULL || tk + r < valid;           // keys past the end contribute nothing
            const float cp = live ? __builtin_amdgcn_rcpf(zp) : 0.0f;
            const float cn = live ? __builtin_amdgcn_rcpf(zn) : 0.0f;
#pragma unroll
            for (int mb = 0; mb < 4; mb++) {
                kp[mb][r] *= cp;
                kn[mb][r] *= cn;
            }
        }
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
            store4(sPKT + (16 * mb + r16) * S::PT + tk, to_bf16x4(kp[mb]));
            store4(sPKT + (64 + 16 * mb + r16) * S::PT + tk, to_bf16x4(kn[mb]));
        }
        if constexpr (KO) return;
        // queries: lane token i, directions 16 mb + 4 g + r
        float a = -INFINITY, b = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 4; mb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float x = acc[1][mb][r] * kLog2e;
                a = fmaxf(a, x);
                b = fmaxf(b, -x);
            }
        a = fmaxf(a, __shfl_xor(a, 16));
        b = fmaxf(b, __shfl_xor(b, 16));
        const float mq = fmaxf(a, __shfl_xor(a, 32)), nq = fmaxf(b, __shfl_xor(b, 32));
        f32x4 qp[4], qn[4];
        float sp = 0.0f, sn = 0.0f;
#pragma unroll
        for (int mb = 0; mb < 4; mb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float x = acc[1][mb][r] * kLog2e;
                qp[mb][r] = exp2_fast(x - mq);
                qn[mb][r] = exp2_fast(-x - nq);
                sp += qp[mb][r];
                sn += qn[mb][r];
            }
        sp += __shfl_xor(sp, 16);
        sn += __shfl_xor(sn, 16);
        const float cq = __builtin_amdgcn_rcpf(sp + __shfl_xor(sp, 32)), cqn = __builtin_amdgcn_rcpf(sn + __shfl_xor(sn, 32));
        bf16x4 pe[4], ne[4];
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
            f32x4 ep, en;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                ep[r] = qp[mb][r] * cq;
                en[r] = qn[mb][r] * cqn;
            }
            pe[mb] = to_bf16x4(ep);
            ne[mb] = to_bf16x4(en);
        }
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
            store8(sPQ + i * S::RQ + feat_pos<true>(32 * hh + 4 * g), cat(pe[2 * hh], pe[2 * hh + 1]));
            store8(sPQ + i * S::RQ + feat_pos<true>(64 + 32 * hh + 4 * g), cat(ne[2 * hh], ne[2 * hh + 1]));
        }
        return;
    }
    {  // keys: phi(k)^T rows 16 mb + r16 and 64 + that, tokens 16 p + 4 g .. + 3
        const int tk = 16 * p + 4 * g;
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
            f32x4 ep, en;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float u = acc[0][mb][r] * kLog2e + bk2[mb];
                ep[r] = exp2_fast(u);
                en[r] = exp2_fast(-u);
                if (!FULL && tk + r >= valid) ep[r] = en[r] = 0.0f;  // keys past the end contribute nothing
            }
            store4(sPKT + (16 * mb + r16) * S::PT + tk, to_bf16x4(ep));
            store4(sPKT + (64 + 16 * mb + r16) * S::PT + tk, to_bf16x4(en));
        }
    }
    if constexpr (!KO) {  // queries: direction blocks 2 h, 2 h + 1 share one 16-byte run of their 32-feature group
        bf16x4 pe[4], ne[4];
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
            f32x4 ep, en;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float u = acc[1][mb][r] * kLog2e + bl2[mb][r];
                ep[r] = exp2_fast(u);
                en[r] = exp2_fast(-u);
            }
            pe[mb] = to_bf16x4(ep);
            ne[mb] = to_bf16x4(en);
        }
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
            store8(sPQ + i * S::RQ + feat_pos<true>(32 * hh + 4 * g), cat(pe[2 * hh], pe[2 * hh + 1]));
            store8(sPQ + i * S::RQ + feat_pos<true>(64 + 32 * hh + 4 * g), cat(ne[2 * hh], ne[2 * hh + 1]));
        }
    }
}

template <bool SM = false, bool KO = false>
__device__ __forceinline__ void cw64_features_any(const unsigned char *xq, const unsigned char *xk, int valid,
                                                  const bf16x8 (&wA)[4][2], const float (&bl2)[4][4],
                                                  const float (&bk2)[4], int p, int g, int r16, bf16_t *sPQ,
                                                  bf16_t *sPKT) {
    if (valid >= CausalWs64Cfg::C)
        cw64_features<true, SM, KO>(xq, xk, valid, wA, bl2, bk2, p, g, r16, sPQ, sPKT);
    else
        cw64_features<false, SM, KO>(xq, xk, valid, wA, bl2, bk2, p, g, r16, sPQ, sPKT);
}

// One score block (query block ib, key block jb) over the 128 features: A^T[j][i] (lane: query
// 16 ib + r16, keys 16 jb + 4 g + r), causal mask on the diagonal block, bf16 into sA, and its
// row sums into normaliser slot `slot` of the queries.
__device__ __forceinline__ void cw64_score_block(const bf16_t *sPQ, const bf16_t *sPKT, bf16_t *sA, float *sDen, int ib,
                                                 int jb, int slot, int g, int r16) {
    using S = CausalWs64Cfg;
    bf16x8 ka[4], qb[4];
    const int lop = (4 * g + (r16 >> 2)) * S::PT + 4 * (r16 & 3);
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        const bf16_t *pk = sPKT + lop + 32 * ks * S::PT + 16 * jb;
        ka[ks] = cat(lds_read_tr(pk), lds_read_tr(pk + 16 * S::PT));
        qb[ks] = load8(sPQ + (16 * ib + r16) * S::RQ + 32 * ks + 8 * g);
    }
    f32x4 a2[2] = {zero4(), zero4()};
#pragma unroll
    for (int ks = 0; ks < 4; ks++) a2[ks & 1] = mfma_bf16(ka[ks], qb[ks], a2[ks & 1]);
    f32x4 a = a2[0] + a2[1];
    if (jb == ib) {
#pragma unroll
        for (int r = 0; r < 4; r++)
            if (4 * g + r > r16) a[r] = 0.0f;
    }
    const bf16x4 ab = to_bf16x4(a);
    float rs = ((float)ab[0] + (float)ab[1]) + ((float)ab[2] + (float)ab[3]);
    store4(sA + (16 * ib + r16) * S::RA + 16 * jb + 4 * g, ab);
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    sDen[(16 * ib + r16) * S::NDEN + slot] = rs;  // the same value in all four lane groups
}

// Producer p's scores of one chunk: p0 blocks (0,0) and (1,1); p1 block (1,0), and zeros for the
// masked block (0,1) and its row-sum slot.  Slots 2 / 3: row sums over key blocks 0 / 1.
__device__ __forceinline__ void cw64_scores(const bf16_t *sPQ, const bf16_t *sPKT, bf16_t *sA, float *sDen, int p,
                                            int g, int r16) {
    using S = CausalWs64Cfg;
    if (p == 0) {
        cw64_score_block(sPQ, sPKT, sA, sDen, 0, 0, 2, g, r16);
        cw64_score_block(sPQ, sPKT, sA, sDen, 1, 1, 3, g, r16);
    } else {
        cw64_score_block(sPQ, sPKT, sA, sDen, 1, 0, 2, g, r16);
        bf16x4 zz;
        zz[0] = zz[1] = zz[2] = zz[3] = (__bf16)0.0f;
        store4(sA + r16 * S::RA + 16 + 4 * g, zz);
        sDen[r16 * S::NDEN + 3] = 0.0f;
    }
}

__device__ __forceinline__ float cw64_den(const float *sDen, int i) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(sDen + i * CausalWs64Cfg::NDEN);
    return (a[0] + a[1]) + (a[2] + a[3]);
}

// Consumer v: finish the outputs of one chunk (held read-out + intra-chunk product, normalise,
// store).  Lane (g, r16) owns token 16 ib + r16, value columns 32 v + 8 g .. + 7.
__device__ __forceinline__ void cw64_output(f32x4 (&numT)[2][2], const bf16_t *sA, const bf16_t *sV,
                                            const float *sDen, int lane_v, bf16_t *__restrict__ yrow0, int valid,
                                            int v, int g, int r16, bool store) {
    using S = CausalWs64Cfg;
    bf16x8 vop[2];
#pragma unroll
    for (int vb = 0; vb < 2; vb++) vop[vb] = operand_down_rows(sV, lane_v, 4 * vb, S::D);
#pragma unroll
    for (int ib = 0; ib < 2; ib++) {
        const int i = 16 * ib + r16;
        const bf16x8 a = load8(sA + i * S::RA + 8 * g);
#pragma unroll
        for (int vb = 0; vb < 2; vb++) numT[ib][vb] = mfma_bf16(vop[vb], a, numT[ib][vb]);
        const float rden = __builtin_amdgcn_rcpf(cw64_den(sDen, i));
        f32x4 o0, o1;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            o0[r] = numT[ib][0][r] * rden;
            o1[r] = numT[ib][1][r] * rden;
        }
        if (store && i < valid)
            store8(yrow0 + (size_t)i * S::D + value_col<2>(v, 0, 4 * g), cat(to_bf16x4(o0), to_bf16x4(o1)));
    }
}

// Inputs of chunk c + 1 (V) and c + 2 (q, k) into the buffers freed by the last chunk; each
// pipeline wave moves its own 1 KB block of each tile.
// ST: no query tiles (the segment-state mode).
template <bool ST = false>
__device__ __forceinline__ void cw64_issue(const WideParams &p, const Dma64Lanes &dl, size_t base, int t_begin,
                                           int t_end, int c, int n, int pw, unsigned char *sm) {
    using S = CausalWs64Cfg;
    if (c + 1 < n) {
        const int t = t_begin + S::C * (c + 1);
        dl.issue<true>(p.v + base, t, min(S::C, t_end - t), pw, sm + S::OFF_V + ((c + 1) % 3) * S::SZ_X);
    }
    if (c + 2 < n) {
        const int t = t_begin + S::C * (c + 2), b = c & 1;
        if (!ST) dl.issue<false>(p.q + base, t, min(S::C, t_end - t), pw, sm + S::OFF_XQ + b * S::SZ_X);
        dl.issue<false>(p.k + base, t, min(S::C, t_end - t), pw, sm + S::OFF_XK + b * S::SZ_X);
    }
}

// SM: the per-half softmax map (no bias; see cw64_features) instead of the Hedgehog map.
// ST: segment-state mode: the keys' features only and the consumers' update alone, from a zero
// state; the segment's aggregate goes to its slot in the d = 64 segment-state pass's image.
template <bool SM = false, bool ST = false>
__global__ __launch_bounds__(512, 1) void causal_ws_kernel_64(WideParams p) {
    using S = CausalWs64Cfg;
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::LDS_BYTES];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int pipe = (w >> 1) & 1, role = w >> 2, idx = w & 1;
    const int pw = 2 * role + idx;  // wave within the pipeline: producers 0, 1, consumers 2, 3
    int pair, s;
    wg_head_segment(p.nseg_grid, pair, s);
    // sequence of this pipeline.  With a multiple of 16 sequences, pair j holds sequences
    // x + 16 m and x + 16 m + 8 (x = j mod 8, m = j / 8): both of XCD x, where the segment-state
    // pass wrote their slots and where this pair's workgroups run.  An odd count leaves the last
    // pipeline repeating the sequence before without writing anything.
    const int bh_raw = p.BH % 16 == 0 ? (pair & 7) + 16 * (pair >> 3) + 8 * pipe : 2 * pair + pipe;
    const bool writes = bh_raw < p.BH;
    const int bh = writes ? bh_raw : bh_raw - 1;
    const int h = bh % p.H;
    const int t_begin = s * p.seg_len;
    const int t_end = min(p.N, t_begin + p.seg_len);
    const size_t base = (size_t)bh * p.N * S::D;
    const int n = t_end > t_begin ? (t_end - t_begin + S::C - 1) / S::C : 0;
    unsigned char *sm = smem + pipe * S::PIPE_BYTES;
    const Dma64Lanes dl(pw, lane);
    auto valid_of = [&](int c) { return min(S::C, t_end - (t_begin + S::C * c)); };
    auto pq_buf = [&](int b) { return reinterpret_cast<bf16_t *>(sm + S::OFF_PQ + b * S::SZ_PQ); };
    auto pk_buf = [&](int b) { return reinterpret_cast<bf16_t *>(sm + S::OFF_PK + b * S::SZ_PK); };
    auto v_buf = [&](int b) { return reinterpret_cast<const bf16_t *>(sm + S::OFF_V + b * S::SZ_X); };
    auto a_buf = [&](int b) { return reinterpret_cast<bf16_t *>(sm + S::OFF_A + b * S::SZ_A); };
    auto den_buf = [&](int b) { return reinterpret_cast<float *>(sm + S::OFF_DEN + b * S::SZ_DEN); };

    unsigned int *psync = reinterpret_cast<unsigned int *>(sm + S::OFF_SYNC);
    if (pw == 0 && lane == 0) *psync = 0u;
    __syncthreads();
    if (role == 0) {
        // producer idx: the staging loads of the prologue (pipeline blocks idx and idx + 2)
#pragma unroll
        for (int hw = 0; hw < 2; hw++) {
            const Dma64Lanes dh(idx + 2 * hw, lane);
            if (n > 0) {
                if (!ST) dh.issue<false>(p.q + base, t_begin, valid_of(0), idx + 2 * hw, sm + S::OFF_XQ);
                dh.issue<false>(p.k + base, t_begin, valid_of(0), idx + 2 * hw, sm + S::OFF_XK);
                dh.issue<true>(p.v + base, t_begin, valid_of(0), idx + 2 * hw, sm + S::OFF_V);
            }
            if (n > 1) {
                if (!ST)
                    dh.issue<false>(p.q + base, t_begin + S::C, valid_of(1), idx + 2 * hw, sm + S::OFF_XQ + S::SZ_X);
                dh.issue<false>(p.k + base, t_begin + S::C, valid_of(1), idx + 2 * hw, sm + S::OFF_XK + S::SZ_X);
            }
        }
        // W operands straight from memory (rows 16 mb + r16, input dims 32 ks + 8 g .. + 7) and
        // the bias of the query rows (16 mb + 4 g + r) and of the key column (16 mb + r16).  The
        // bias is loaded without a branch (from W in place of a missing bias, then replaced by
        // zero): a test per element would wait for each of these loads before issuing the next.
        bf16x8 wA[4][2];
        float bl2[4][4], bk2[4];
        const bf16_t *Wh = p.W + (size_t)h * 64 * 64;
        const bool has_b = p.b != nullptr;
        const bf16_t *bsrc = has_b ? p.b + (size_t)h * 64 : Wh;  // W has 64 x 64 entries per head
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
#pragma unroll
            for (int ks = 0; ks < 2; ks++) wA[mb][ks] = load8(Wh + (size_t)(16 * mb + r16) * 64 + 32 * ks + 8 * g);
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float bv = bf16_bits_to_float(bsrc[16 * mb + 4 * g + r]) * kLog2e;
                bl2[mb][r] = has_b ? bv : 0.0f;
            }
            const float bv = bf16_bits_to_float(bsrc[16 * mb + r16]) * kLog2e;
            bk2[mb] = has_b ? bv : 0.0f;
        }
        producer_barrier(psync, 2, lane);
        if (n > 0)
            cw64_features_any<SM, ST>(sm + S::OFF_XQ, sm + S::OFF_XK, valid_of(0), wA, bl2, bk2, idx, g, r16,
                                      pq_buf(0), pk_buf(0));
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int c = 0; c < n; c++) {
            cw64_issue<ST>(p, dl, base, t_begin, t_end, c, n, pw, sm);
            const int b2 = c & 1;
            if (!ST) cw64_scores(pq_buf(b2), pk_buf(b2), a_buf(b2), den_buf(b2), idx, g, r16);
            if (c + 1 < n)
                cw64_features_any<SM, ST>(sm + S::OFF_XQ + (b2 ^ 1) * S::SZ_X, sm + S::OFF_XK + (b2 ^ 1) * S::SZ_X,
                                          valid_of(c + 1), wA, bl2, bk2, idx, g, r16, pq_buf(b2 ^ 1), pk_buf(b2 ^ 1));
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        return;
    }
    // Consumer v = idx: value columns value_col<2>(v, vb, c) of S for all 128 features, z rows
    // of feature blocks 4 v .. 4 v + 3.
    const int v = idx;
    f32x4 sacc[8][2];
    f32x4 zacc[4];
    {
#pragma unroll
        for (int fb = 0; fb < 8; fb++) sacc[fb][0] = sacc[fb][1] = zero4();
#pragma unroll
        for (int zb = 0; zb < 4; zb++) zacc[zb] = zero4();
        if (!ST && p.S_in) {
            const float *Si = p.S_in + (size_t)bh * p.in_bh_stride * S::DP * S::D;
            const float *zi = p.z_in + (size_t)bh * p.in_bh_stride * S::DP;
#pragma unroll
            for (int fb = 0; fb < 8; fb++)
#pragma unroll
                for (int vb = 0; vb < 2; vb++) {
                    const int nn = value_col<2>(v, vb, r16);
#pragma unroll
                    for (int r = 0; r < 4; r++) sacc[fb][vb][r] = Si[(size_t)(16 * fb + 4 * g + r) * S::D + nn];
                }
#pragma unroll
            for (int zb = 0; zb < 4; zb++)
#pragma unroll
                for (int r = 0; r < 4; r++) zacc[zb][r] = zi[16 * (4 * v + zb) + 4 * g + r];
        }
        int t0 = 0, t1 = 0;  // slots to add
        if (!ST && s > 0 && p.slot_mode == 1) t0 = s, t1 = s + 1;
        if (!ST && s > 0 && p.slot_mode == 3) t0 = 0, t1 = s;
        // slot image of the d = 64 segment-state pass: value column nn, feature block fb of wave
        // nn / 16 sits in piece (nn / 16) 4 + fb / 2, half fb % 2, lane 16 g + nn % 16
        int lsrc[2], esrc[2];
#pragma unroll
        for (int vb = 0; vb < 2; vb++) {
            const int nn = value_col<2>(v, vb, r16);
            lsrc[vb] = 16 * g + (nn & 15);
            esrc[vb] = (nn >> 4) * 4;
        }
        for (int t = t0; t < t1; t++) {
            const size_t sl = (size_t)bh * p.slot_bh_stride + t;
            const float *zs = p.z_slots + sl * S::DP;
            const float *img = p.S_slots + sl * S::DP * S::D;
            f32x4 zslot[4], raw[8][2];
#pragma unroll
            for (int zb = 0; zb < 4; zb++) zslot[zb] = *reinterpret_cast<const f32x4 *>(zs + 16 * (4 * v + zb) + 4 * g);
#pragma unroll
            for (int fb = 0; fb < 8; fb++)
#pragma unroll
                for (int vb = 0; vb < 2; vb++) raw[fb][vb] = *slot_piece(img, esrc[vb] + (fb >> 1), fb & 1, lsrc[vb]);
#pragma unroll
            for (int fb = 0; fb < 8; fb++)
#pragma unroll
                for (int vb = 0; vb < 2; vb++) sacc[fb][vb] += raw[fb][vb];
#pragma unroll
            for (int zb = 0; zb < 4; zb++) zacc[zb] += zslot[zb];
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const int r0 = 8 * g + (r16 >> 2);
    const int lane_v = r0 * S::D + 8 * v_pos64(r0, 4 * v + (r16 & 3));
    const bf16x8 ones = ones_bf16x8();
    if constexpr (ST) {
        // the update alone: S += phi(K)^T V and z += phi(K)^T 1 per chunk, as in the loop below
        for (int c = 0; c < n; c++) {
            cw64_issue<true>(p, dl, base, t_begin, t_end, c, n, pw, sm);
            const bf16_t *sPK = pk_buf(c & 1);
            const bf16_t *sV = v_buf(c % 3);
            bf16x8 vop[2], an[2];
#pragma unroll
            for (int vb = 0; vb < 2; vb++) vop[vb] = operand_down_rows(sV, lane_v, 4 * vb, S::D);
#pragma unroll
            for (int j = 0; j < 2; j++) an[j] = load8(sPK + (16 * j + r16) * S::PT + 8 * g);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                const bf16x8 ac[2] = {an[0], an[1]};
                if (ks < 3) {
#pragma unroll
                    for (int j = 0; j < 2; j++) an[j] = load8(sPK + (32 * (ks + 1) + 16 * j + r16) * S::PT + 8 * g);
                }
#pragma unroll
                for (int j = 0; j < 2; j++)
#pragma unroll
                    for (int vb = 0; vb < 2; vb++)
                        sacc[2 * ks + j][vb] = mfma_bf16(ac[j], vop[vb], sacc[2 * ks + j][vb]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int zb = 0; zb < 4; zb++)
                zacc[zb] = mfma_bf16(load8(sPK + (16 * (4 * v + zb) + r16) * S::PT + 8 * g), ones, zacc[zb]);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        if (!writes) return;
        // slot s, in the pieces the slot sum above reads back
        const size_t sl = (size_t)bh * p.slot_bh_stride + s;
        float *img = p.S_slots + sl * S::DP * S::D;
#pragma unroll
        for (int vb = 0; vb < 2; vb++) {
            const int nn = value_col<2>(v, vb, r16);
#pragma unroll
            for (int fb = 0; fb < 8; fb++) *slot_piece(img, (nn >> 4) * 4 + (fb >> 1), fb & 1, 16 * g + (nn & 15)) = sacc[fb][vb];
        }
        if (r16 == 0) {
            float *zs = p.z_slots + sl * S::DP;
#pragma unroll
            for (int zb = 0; zb < 4; zb++)
#pragma unroll
                for (int r = 0; r < 4; r++) zs[16 * (4 * v + zb) + 4 * g + r] = zacc[zb][r];
        }
        return;
    }

    f32x4 numT[2][2];
#pragma unroll
    for (int ib = 0; ib < 2; ib++) numT[ib][0] = numT[ib][1] = zero4();
    bf16_t *ybase = p.y + base;

    for (int c = 0; c < n; c++) {
        cw64_issue(p, dl, base, t_begin, t_end, c, n, pw, sm);
        const int b2 = c & 1;
        const bf16_t *sPQ = pq_buf(b2);
        const bf16_t *sPK = pk_buf(b2);
        const bf16_t *sVp = v_buf((c + 2) % 3);
        const bf16_t *sAp = a_buf(b2 ^ 1);
        const float *sDp = den_buf(b2 ^ 1);
        bf16x8 vp[2], ao[2];
#pragma unroll
        for (int vb = 0; vb < 2; vb++) vp[vb] = operand_down_rows(sVp, lane_v, 4 * vb, S::D);
#pragma unroll
        for (int ib = 0; ib < 2; ib++) ao[ib] = load8(sAp + (16 * ib + r16) * S::RA + 8 * g);
        const bf16_t *sV = v_buf(c % 3);
        bf16x8 vop[2];
#pragma unroll
        for (int vb = 0; vb < 2; vb++) vop[vb] = operand_down_rows(sV, lane_v, 4 * vb, S::D);
        bf16x8 qn[2], an[2];
        auto load_step = [&](int ks, bf16x8(&qo)[2], bf16x8(&ao2)[2]) {
#pragma unroll
            for (int ib = 0; ib < 2; ib++) qo[ib] = load8(sPQ + (16 * ib + r16) * S::RQ + 32 * ks + 8 * g);
#pragma unroll
            for (int j = 0; j < 2; j++) ao2[j] = load8(sPK + (32 * ks + 16 * j + r16) * S::PT + 8 * g);
        };
        load_step(0, qn, an);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 nt[2][2];
#pragma unroll
        for (int ib = 0; ib < 2; ib++) nt[ib][0] = nt[ib][1] = zero4();
        float dsum[2];
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            bf16x8 qc[2] = {qn[0], qn[1]}, ac[2] = {an[0], an[1]};
            if (ks < 3) load_step(ks + 1, qn, an);
            if (ks == 0) {  // intra-chunk product of chunk c - 1
#pragma unroll
                for (int ib = 0; ib < 2; ib++)
#pragma unroll
                    for (int vb = 0; vb < 2; vb++) numT[ib][vb] = mfma_bf16(vp[vb], ao[ib], numT[ib][vb]);
            }
            if (ks == 1) {  // its normaliser
#pragma unroll
                for (int ib = 0; ib < 2; ib++) dsum[ib] = cw64_den(sDp, 16 * ib + r16);
            }
            bf16x8 sb[2];
#pragma unroll
            for (int vb = 0; vb < 2; vb++) sb[vb] = acc_pair_to_operand(sacc[2 * ks][vb], sacc[2 * ks + 1][vb]);
#pragma unroll
            for (int ib = 0; ib < 2; ib++)
#pragma unroll
                for (int vb = 0; vb < 2; vb++) nt[ib][vb] = mfma_bf16(sb[vb], qc[ib], nt[ib][vb]);
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int vb = 0; vb < 2; vb++) sacc[2 * ks + j][vb] = mfma_bf16(ac[j], vop[vb], sacc[2 * ks + j][vb]);
            if (ks == 2 && c > 0 && writes) {  // outputs of chunk c - 1 (every token of it is valid)
                bf16_t *yrow0 = ybase + (size_t)(t_begin + S::C * (c - 1)) * S::D;
#pragma unroll
                for (int ib = 0; ib < 2; ib++) {
                    const float rden = __builtin_amdgcn_rcpf(dsum[ib]);
                    f32x4 o0, o1;
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        o0[r] = numT[ib][0][r] * rden;
                        o1[r] = numT[ib][1][r] * rden;
                    }
                    store8(yrow0 + (size_t)(16 * ib + r16) * S::D + value_col<2>(v, 0, 4 * g),
                           cat(to_bf16x4(o0), to_bf16x4(o1)));
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int ib = 0; ib < 2; ib++) {
            numT[ib][0] = nt[ib][0];
            numT[ib][1] = nt[ib][1];
        }
        f32x4 dacc[2] = {zero4(), zero4()};
        {
            const bf16_t *sPQz = sPQ + 64 * v;  // K steps 2 v, 2 v + 1
#pragma unroll
            for (int kz = 0; kz < 2; kz++) {
                const bf16x8 zop = acc_pair_to_operand(zacc[2 * kz], zacc[2 * kz + 1]);
#pragma unroll
                for (int ib = 0; ib < 2; ib++)
                    dacc[ib] = mfma_bf16(zop, load8(sPQz + (16 * ib + r16) * S::RQ + 32 * kz + 8 * g), dacc[ib]);
            }
        }
        // every row of dacc holds the token's partial: all four lane groups write the same value
        float *sDen = den_buf(b2);
        sDen[r16 * S::NDEN + v] = dacc[0][0];
        sDen[(16 + r16) * S::NDEN + v] = dacc[1][0];
#pragma unroll
        for (int zb = 0; zb < 4; zb++)
            zacc[zb] = mfma_bf16(load8(sPK + (16 * (4 * v + zb) + r16) * S::PT + 8 * g), ones, zacc[zb]);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    if (n > 0)
        cw64_output(numT, a_buf((n - 1) & 1), v_buf((n - 1) % 3), den_buf((n - 1) & 1), lane_v,
                    ybase + (size_t)(t_begin + S::C * (n - 1)) * S::D, valid_of(n - 1), v, g, r16, writes);
    if (writes && p.S_out && s == p.nseg_grid - 1) {
        float *So = p.S_out + (size_t)bh * S::DP * S::D;
        float *zo = p.z_out + (size_t)bh * S::DP;
#pragma unroll
        for (int fb = 0; fb < 8; fb++)
#pragma unroll
            for (int vb = 0; vb < 2; vb++) {
                const int nn = value_col<2>(v, vb, r16);
#pragma unroll
                for (int r = 0; r < 4; r++) So[(size_t)(16 * fb + 4 * g + r) * S::D + nn] = sacc[fb][vb][r];
            }
        if (r16 == 0) {
#pragma unroll
            for (int zb = 0; zb < 4; zb++)
#pragma unroll
                for (int r = 0; r < 4; r++) zo[16 * (4 * v + zb) + 4 * g + r] = zacc[zb][r];
        }
    }
}

// Stand-alone feature map: each workgroup maps `cpw` chunks of 64 tokens of one head and
// writes phi [token][2d] through an LDS tile so that global stores are full 16-byte rows.
template <int D>
__global__ __launch_bounds__(WideCfg<D>::NT, WideCfg<D>::MIN_WG_PER_CU) void fm_hedgehog_kernel(const bf16_t *__restrict__ x,
                                                                        const bf16_t *__restrict__ W,
                                                                        const bf16_t *__restrict__ b,
                                                                        bf16_t *__restrict__ phi, int H, int N,
                                                                        int cpw, int wg_per_bh) {
    using K = WideCfg<D>;
    __shared__ __attribute__((aligned(16))) bf16_t sPhi[K::C * K::RQ];
    __shared__ __attribute__((aligned(16))) unsigned char sStage[K::SZ_X];
    const int tid = threadIdx.x;
    // wave index as a scalar: role branches on it stay scalar (never exec-masked around MFMAs)
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int th = w / K::NDQ, dq = w % K::NDQ;
    const int bh = blockIdx.x / wg_per_bh, part = blockIdx.x % wg_per_bh;
    const int h = bh % H;
    bf16x8 wA[K::LB][K::KSD];
    float bl2[K::LB][4];
    load_directions<D>(W, b, h, dq, g, r16, wA, bl2);
    const bf16_t *xh = x + (size_t)bh * N * D;
    bf16_t *ph = phi + (size_t)bh * N * K::DP;
    for (int c = 0; c < cpw; c++) {
        const int t0 = (part * cpw + c) * K::C;
        if (t0 >= N) break;
        const int valid = min(K::C, N - t0);
        stage_x<D, K::C>(xh, t0, valid, w, lane, sStage);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        phi_chunk<D, K::C, false, true, false>(sStage, valid, wA, bl2, th, dq, g, r16, sPhi, K::RQ);
        __syncthreads();
        constexpr int P8 = K::DP / 8;
        for (int pi = tid; pi < K::C * P8; pi += K::NT) {
            const int i = pi / P8, c8 = pi % P8;
            if (i < valid) store8(ph + (size_t)(t0 + i) * K::DP + 8 * c8, load8(sPhi + i * K::RQ + 8 * c8));
        }
        __syncthreads();
    }
}

template <int D>
static hipError_t launch_fm_d(const bf16_t *x, const bf16_t *W, const bf16_t *b, bf16_t *phi, int BH, int H, int N,
                              hipStream_t st) {
    using K = WideCfg<D>;
    const long nch = (N + K::C - 1) / K::C;
    // enough workgroups to fill the chip, several chunks each to amortise loading W
    long cpw = ((long)BH * nch) / 1024;
    if (cpw < 1) cpw = 1;
    if (cpw > 8) cpw = 8;
    const long wpb = (nch + cpw - 1) / cpw;
    hipLaunchKernelGGL((fm_hedgehog_kernel<D>), dim3((unsigned)(BH * wpb)), dim3(K::NT), 0, st, x, W, b, phi, H, N,
                       (int)cpw, (int)wpb);
    return hipGetLastError();
}

hipError_t launch_featuremap_hedgehog_bf16(int d, const bf16_t *x, const bf16_t *W, const bf16_t *b, bf16_t *phi,
                                           int BH, int H, int N, hipStream_t st) {
    switch (d) {
    case 16: return launch_fm_d<16>(x, W, b, phi, BH, H, N, st);
    case 32: return launch_fm_d<32>(x, W, b, phi, BH, H, N, st);
    case 64: return launch_fm_d<64>(x, W, b, phi, BH, H, N, st);
    case 128: return launch_fm_d<128>(x, W, b, phi, BH, H, N, st);
    default: return hipErrorInvalidValue;
    }
}

// Scan of the segment slots of each sequence, in place: mode 0 (causal) leaves in slot s the
// exclusive prefix (the sum of slots 0 .. s - 1) for s >= 1 and in slot nseg - 1 the sum of the
// first nseg - 1; mode 1 (bidirectional) leaves the total of all nseg slots in slot 0.  One
// thread per 16 bytes of a slot (S and z alike); each thread loads eight slots before it adds or
// stores any, so the loads of a sequence are in flight together; the slot layout does not matter
// (every slot of a sequence has the same one).  Workgroup b works on a
// sequence of XCD b mod 8 when BH is a multiple of 8, the XCD whose workgroups wrote its slots.
template <int D>
__global__ __launch_bounds__(256) void slot_scan_kernel(float *__restrict__ S, float *__restrict__ z, int BH, int nseg,
                                                        int mode) {
    constexpr int PS = 2 * D * D / 4, PZ = 2 * D / 4;  // f32x4 per slot: S, z
    constexpr int WPH = (PS + PZ + 255) / 256;           // workgroups per sequence
    const int b = blockIdx.x;
    int bh, part;
    if (BH % 8 == 0) {
        const int j = b >> 3;
        bh = (b & 7) + 8 * (j / WPH);
        part = j % WPH;
    } else {
        bh = b / WPH;
        part = b % WPH;
    }
    const int e = part * 256 + threadIdx.x;
    if (bh >= BH || e >= PS + PZ) return;
    f32x4 *base;
    long stride;
    if (e < PS) {
        base = reinterpret_cast<f32x4 *>(S) + (long)bh * nseg * PS + e;
        stride = PS;
    } else {
        base = reinterpret_cast<f32x4 *>(z) + (long)bh * nseg * PZ + (e - PS);
        stride = PZ;
    }
    const int nin = mode == 0 ? nseg - 1 : nseg;
    f32x4 run = zero4();
    for (int s0 = 0; s0 < nin; s0 += 8) {
        f32x4 a[8];
#pragma unroll
        for (int i = 0; i < 8; i++)
            if (s0 + i < nin) a[i] = base[(s0 + i) * stride];
#pragma unroll
        for (int i = 0; i < 8; i++)
            if (s0 + i < nin) {
                if (mode == 0 && s0 + i > 0) base[(s0 + i) * stride] = run;
                run += a[i];
            }
    }
    base[mode == 0 ? (long)(nseg - 1) * stride : 0] = run;
}

hipError_t launch_slot_scan(int d, float *S_slots, float *z_slots, int BH, int nseg, int mode, hipStream_t st) {
    const long per = ((2L * d * d / 4 + 2L * d / 4) + 255) / 256;
    const unsigned grid = (unsigned)(BH * per);
    switch (d) {
    case 16: hipLaunchKernelGGL(slot_scan_kernel<16>, dim3(grid), dim3(256), 0, st, S_slots, z_slots, BH, nseg, mode); break;
    case 32: hipLaunchKernelGGL(slot_scan_kernel<32>, dim3(grid), dim3(256), 0, st, S_slots, z_slots, BH, nseg, mode); break;
    case 64: hipLaunchKernelGGL(slot_scan_kernel<64>, dim3(grid), dim3(256), 0, st, S_slots, z_slots, BH, nseg, mode); break;
    case 128: hipLaunchKernelGGL(slot_scan_kernel<128>, dim3(grid), dim3(256), 0, st, S_slots, z_slots, BH, nseg, mode); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D>
static hipError_t launch_wide_d(int mode, const WideParams &p, int grid, hipStream_t st) {
    using K = WideCfg<D>;
    switch (mode) {
    case WM_STATE:
        // the softmax maps: the chunked pass's pipeline in its segment-state mode (its producers
        // normalise without workgroup barriers; at B1 H32 N4096 d128 and B8 H12 N1024 d64 it takes
        // 11 % and 9 % less time per call than the all-wave segment-state pass with the softmax)
        if (D == 128 && p.softmax)
            hipLaunchKernelGGL((causal_ws_kernel_128<true, true>), dim3(grid), dim3(CausalWsCfg::NT), 0, st, p);
        else if (D == 64 && p.softmax)  // likewise at d = 64, two sequences per workgroup
            hipLaunchKernelGGL((causal_ws_kernel_64<true, true>), dim3((unsigned)((p.BH + 1) / 2 * p.nseg_grid)),
                               dim3(CausalWs64Cfg::NT), 0, st, p);
        else if (D == 128 || D == 64)
            hipLaunchKernelGGL((state_sym_kernel<D == 128 ? 128 : 64>), dim3(grid),
                               dim3(StateSymCfg<D == 128 ? 128 : 64>::NT), 0, st, p);
        else
            hipLaunchKernelGGL((wide_kernel<D, WM_STATE>), dim3(grid), dim3(K::NT), 0, st, p);
        break;
    case WM_CAUSAL:
        if (D == 128 && p.softmax)
            hipLaunchKernelGGL(causal_ws_kernel_128<true>, dim3(grid), dim3(CausalWsCfg::NT), 0, st, p);
        else if (D == 128)
            hipLaunchKernelGGL(causal_ws_kernel_128<false>, dim3(grid), dim3(CausalWsCfg::NT), 0, st, p);
        else if (D == 64 && p.softmax)  // two sequences per workgroup
            hipLaunchKernelGGL(causal_ws_kernel_64<true>, dim3((unsigned)((p.BH + 1) / 2 * p.nseg_grid)),
                               dim3(CausalWs64Cfg::NT), 0, st, p);
        else if (D == 64)
            hipLaunchKernelGGL(causal_ws_kernel_64<false>, dim3((unsigned)((p.BH + 1) / 2 * p.nseg_grid)),
                               dim3(CausalWs64Cfg::NT), 0, st, p);
        else
            hipLaunchKernelGGL((wide_kernel<D, WM_CAUSAL>), dim3(grid), dim3(K::NT), 0, st, p);
        break;
    default:
        hipLaunchKernelGGL((wide_kernel<D, WM_READOUT>), dim3(grid), dim3(K::NT), 0, st, p);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_wide(int d, int mode, const WideParams &p, int grid, hipStream_t st) {
    // the softmax map runs on the d = 64 and 128 segment-state and causal kernels only
    if (p.softmax && !((d == 128 || d == 64) && (mode == WM_STATE || mode == WM_CAUSAL))) return hipErrorInvalidValue;
    switch (d) {
    case 16: return launch_wide_d<16>(mode, p, grid, st);
    case 32: return launch_wide_d<32>(mode, p, grid, st);
    case 64: return launch_wide_d<64>(mode, p, grid, st);
    case 128: return launch_wide_d<128>(mode, p, grid, st);
    default: return hipErrorInvalidValue;
    }
}

template <int D>
constexpr int wide_lds_max() {
    constexpr int a = WideCfg<D, wide_chunk(D, WM_STATE), WM_STATE>::LDS_BYTES;
    constexpr int c = WideCfg<D, wide_chunk(D, WM_CAUSAL), WM_CAUSAL>::LDS_BYTES;
    constexpr int r = WideCfg<D, wide_chunk(D, WM_READOUT), WM_READOUT>::LDS_BYTES;
    return a > c ? (a > r ? a : r) : (c > r ? c : r);
}

int wide_wgs_per_cu(int d) {
    int lds = 0;
    switch (d) {
    case 16: lds = wide_lds_max<16>(); break;
    case 32: lds = wide_lds_max<32>(); break;
    case 64: lds = wide_lds_max<64>(); break;
    case 128: lds = wide_lds_max<128>(); break;
    default: return 1;
    }
    int n = (160 * 1024) / lds;
    if (d == 128) n = 1;  // 8 waves per workgroup already fill the CU
    return n < 1 ? 1 : (n > 4 ? 4 : n);
}

}  // namespace hh
