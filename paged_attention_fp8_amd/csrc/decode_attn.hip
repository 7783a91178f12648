// decode_attn.hip -- decode-phase paged attention over an e4m3 (or bf16) KV
// cache, converting on read, with split-K partitions (merged by
// splitk_combine.hip).
//
// What is computed: Cloudflare, "Smaller, faster, safer: running Kimi and GLM
// at scale", section "KV 缓存量化" (KV cache quantization) -- decode reads a
// KV cache stored as FP8 e4m3 and the attention kernel converts the format as
// it reads; a BF16-cache kernel is kept for direct comparison.  Pages follow
// the per-sequence logical-to-physical mapping of paged attention (remio.ai
// analysis of the post, section on shared KV cache safety).  A request
// aborted by the separate page-tag check (section "共享 KV 缓存保护") is
// neither read nor computed: its output is 0 with lse = -inf.
//
// gfx950 design (the kernels the pages measured were written for H200):
//  * one work-group = 4 wave64s = one (request, KV head, split); the split's
//    tokens are dealt to the waves in tiles of 64 tokens (32 for bf16 pools,
//    so that a tile is 16 KB of K+V either way) and the four partial softmax
//    states are merged through LDS at the end.  In the balanced partition a
//    work-group instead takes an equal range of all requests' pages of its
//    KV head and runs the same per-range code on each request piece in it;
//  * every lane issues 16-byte loads; a wave keeps about one tile (16 KB) in
//    flight at all times with a single register buffer: the next tile's K
//    loads go out as soon as Q.K^T has consumed this tile's K, its V loads as
//    soon as P.V has consumed this tile's V; page ids arrive through scalar
//    loads a tile ahead, so they never queue behind the vector loads;
//  * Q.K^T and P.V run on 16x16x32 MFMAs and the whole query group shares
//    one K/V tile held in registers.  Q.K^T takes the tile's tokens as rows
//    and the group's heads as columns (K decoded exactly to bf16; Q is bf16
//    already); P.V takes head dims as rows (V exact in bf16, P split into a
//    bf16 high and low part; with at most 8 heads in the group the low part
//    rides in the MFMA columns the group leaves free, otherwise it takes a
//    second MFMA).  Token order inside a tile is permuted so that the scores
//    an MFMA leaves in a lane are exactly the P operand that lane feeds to
//    the next MFMA, and the head a lane owns never changes: the online
//    softmax needs two cross-lane max exchanges per tile and no other data
//    movement;
//  * one query head per KV head (G == 1) takes the same MFMA kernels with
//    one live column: the matrix cores have the idle columns to spare, and
//    the tile's conversions and loads are what they are at any G, whereas
//    the same dot products on FMAs kept the VALU too busy to stream;
//  * every kernel has an APPEND instantiation that also writes the step's new
//    token (the append taken into the attention launch).
// Arithmetic: scores and outputs accumulate in fp32, softmax in the exp2
// domain; the result is exact up to fp32 rounding.
#include "attn_params.hpp"
#include "pafp8_append.hpp"
#include "pafp8_device.hpp"

namespace pafp8 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kNegInf = -__builtin_huge_valf();

// Tokens [t0, t1) a work-group covers, and the request's verdict.
struct SplitRange {
    int64_t t0, t1;
    int64_t p_last;  // index of the split's last page
    int state;       // 0 = compute, 1 = aborted (0 / -inf), 2 = invalid (NaN)
};

// Tokens of splits s .. s + nparts - 1 of request b (clipped to its length).
__device__ __forceinline__ SplitRange split_range(const AttnParams &p, int b, int s, int nparts = 1)
{
    SplitRange r{0, 0, 0, 0};
    if (p.req_status != nullptr && p.req_status[b] != 0) {
        r.state = 1;
        return r;
    }
    const int64_t L = p.context_lens[b];
    const int64_t cap = static_cast<int64_t>(p.max_pages) << p.log2_page;
    if (L < 0 || L > cap) {
        r.state = 2;
        return r;
    }
    const int64_t n_pages = (L + (int64_t{1} << p.log2_page) - 1) >> p.log2_page;
    const int64_t p0 = static_cast<int64_t>(s) * p.pages_per_split;
    int64_t p1 = p0 + static_cast<int64_t>(nparts) * p.pages_per_split;
    if (p1 > n_pages)
        p1 = n_pages;
    if (p0 >= p1)
        return r;  // nothing to attend in this split
    r.t0 = p0 << p.log2_page;
    r.t1 = p1 << p.log2_page;
    if (r.t1 > L)
        r.t1 = L;
    r.p_last = p1 - 1;
    return r;
}

// The append taken into the attention launch: the one work-group of a
// (request, KV head) whose tokens end at the request's last token writes that
// token first (thread d, head dim d; nothing when its page lies outside the
// pool), and the work-group barrier orders the stores before any of its waves
// loads the tile that holds them.  No other work-group reads that slot.
// The token's V bytes land one in each of D rows of its segment; written
// while the rest of the GPU streams, such scattered partial-line stores slow
// the launch when every work-group of a large batch makes them (one request
// per work-group), so the fused launch pays off where launches dominate.
template <bool BF16, int D>
__device__ __forceinline__ void append_new_token(const AttnParams &p, int b, int g, int64_t L)
{
    const int64_t pos = L - 1;
    const int32_t page = p.page_table[static_cast<int64_t>(b) * p.max_pages + (pos >> p.log2_page)];
    if (page >= 0 && page < p.num_pages) {
        const int slot = static_cast<int>(pos & ((int64_t{1} << p.log2_page) - 1));
        for (int d = threadIdx.x; d < D; d += kThreads) {
            const int64_t src = (static_cast<int64_t>(b) * p.num_kv_heads + g) * D + d;
            append_token_element<BF16, D, true>(const_cast<uint8_t *>(p.k_pool), const_cast<uint8_t *>(p.v_pool),
                                          page, p.num_kv_heads, g, p.log2_page, slot, d, p.k_new[src],
                                          p.v_new[src], BF16 ? 1.0f : p.k_scale[g],
                                          BF16 ? 1.0f : p.v_scale[g]);
        }
    }
    __syncthreads();
}

// Physical pages of the four token groups of a tile (group q covers tokens
// T0 + q*tpg .. + tpg, always inside one page).  The page ids are
// wave-uniform and come in through scalar loads; they are fetched a tile ahead
// and only checked (pages_ok) when the tile's loads are issued, so the fetch
// never waits for its own result.
struct TilePages {
    int32_t pid[4];
};

// A request's page-table row, read through the constant address space: the
// table does not change during a launch, and saying so keeps its wave-uniform
// reads on the scalar path even in kernels that also write the pool (the
// append taken into the launch), where the compiler could otherwise not rule
// out that the stores change the table and would issue vector loads, which
// queue behind the tile loads and stall the pipeline.
typedef const __attribute__((address_space(4))) int32_t *page_row_t;

__device__ __forceinline__ page_row_t page_row(const AttnParams &p, int b)
{
    return (page_row_t)(p.page_table + static_cast<int64_t>(b) * p.max_pages);
}

template <bool ONE_PAGE = false>
__device__ __forceinline__ TilePages fetch_pages(page_row_t __restrict__ row, int64_t T0,
                                                 int tpg, int log2_page, int64_t p_last)
{
    TilePages t;
    if constexpr (ONE_PAGE) {
        // the whole tile lies in one page
        int64_t idx = T0 >> log2_page;
        if (idx > p_last)
            idx = p_last;
        t.pid[0] = t.pid[1] = t.pid[2] = t.pid[3] = row[idx];
        return t;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        int64_t idx = (T0 + q * tpg) >> log2_page;
        if (idx > p_last)
            idx = p_last;  // past the split (or no such tile): any page of the split is safe
        t.pid[q] = row[idx];
    }
    return t;
}

// Replace page ids outside the pool by page 0 and record that it happened.
__device__ __forceinline__ TilePages pages_ok(TilePages t, int num_pages, int &bad)
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const bool ok = t.pid[q] >= 0 && t.pid[q] < num_pages;
        bad |= ok ? 0 : 1;
        t.pid[q] = ok ? t.pid[q] : 0;
    }
    return t;
}

// pid[q] for a per-lane q in 0..3, as register arithmetic (a select chain
// would be turned into a lookup table in scratch memory).
__device__ __forceinline__ int32_t select4(int q, const TilePages &t)
{
    const int32_t m1 = -(q & 1), m2 = -((q >> 1) & 1);
    const int32_t a = t.pid[0] ^ ((t.pid[0] ^ t.pid[1]) & m1);
    const int32_t b = t.pid[2] ^ ((t.pid[2] ^ t.pid[3]) & m1);
    return a ^ ((a ^ b) & m2);
}

// keep the first n bytes (n in [0, 16]) of a 16-byte register
__device__ __forceinline__ u32x4 keep_bytes(u32x4 w, int n)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = n - 4 * i;  // bytes of dword i to keep
        const uint32_t m = k >= 4 ? 0xFFFFFFFFu : (k <= 0 ? 0u : ((1u << (8 * k)) - 1u));
        w[i] &= m;
    }
    return w;
}

// ===========================================================================
// MFMA path (every query group size, 1 to 16)
// ===========================================================================
template <bool BF16, int D>
struct Geo {
    static constexpr int E = BF16 ? 2 : 1;          // bytes per element
    static constexpr int TT = BF16 ? 32 : 64;       // tokens per wave tile
    static constexpr int TPG = TT / 4;              // tokens per lane group (lane / 16)
    static constexpr int NJ = TT / 16;              // Q.K^T MFMAs along tokens
    static constexpr int NC = D / 32;               // Q.K^T MFMAs along the head dim
    static constexpr int NDT = D / 16;              // P.V MFMAs along the head dim
    static constexpr int NPC = TT / 32;             // P.V MFMAs along tokens
    static constexpr int KL = (D / 4) * E / 16;     // 16-byte K loads per lane per token row
    static constexpr int LOG2_TT = BF16 ? 5 : 6;
    static constexpr int LOG2_TPG = LOG2_TT - 2;
    static_assert(TPG * E == 16, "a lane group's V run must be one 16-byte load");
    static_assert((1 << LOG2_TT) == TT, "tile size");
};

template <bool BF16, int D>
struct MfmaTile {
    u32x4 k[Geo<BF16, D>::NJ][Geo<BF16, D>::KL];
    u32x4 v[Geo<BF16, D>::NDT];
};

template <bool BF16, int D>
struct MfmaCtx {
    const uint8_t *k_head;  // k_pool + g * head block
    const uint8_t *v_head;
    int64_t page_bytes;     // bytes of one page of one pool (all heads)
    int log2_page;
    int lane_r, lane_g;     // lane % 16, lane / 16
};

// 16-byte KV loads.  Every K and V line a tile touches is consumed whole by
// the wave's own load steps, so the loads stream past the caches.
__device__ __forceinline__ u32x4 load16_kv(const void *p)
{
    return load16_stream(p);
}

// Pool block layout (per page and KV head; see include/pafp8.h): blocks are
// cut into segments of min(P, TT) tokens -- exactly one wave tile when the
// page holds one.  K: token TPG*s + 4j + a of a segment keeps its 16-byte
// chunk q*KL + l at chunk ((j*KL + l)*4 + q)*(4*NS) + 4s + a (NS = segment /
// TPG), which is precisely the chunk lane 16q + 4s + a loads in step (j, l):
// every K load step of a tile reads one contiguous run.  V: a segment is
// [D][segment tokens], so a V load step reads 16 consecutive 64-byte rows.
//
// BIG (page >= tile): the tile is one whole segment of one page, so the page
// base is wave-uniform and each load step is 1 KB at a compile-time offset.
template <bool BF16, int D, bool BIG>
__device__ __forceinline__ void mfma_load_k(MfmaTile<BF16, D> &t, const MfmaCtx<BF16, D> &c,
                                            int64_t T0, const TilePages &pg)
{
    using G_ = Geo<BF16, D>;
    if constexpr (BIG) {
        const int seg = static_cast<int>(T0 & ((int64_t{1} << c.log2_page) - 1)) >> G_::LOG2_TT;
        const uint8_t *kp = c.k_head + static_cast<int64_t>(pg.pid[0]) * c.page_bytes +
                            seg * (G_::TT * D * G_::E) + (c.lane_g * 16 + c.lane_r) * 16;
#pragma unroll
        for (int j = 0; j < G_::NJ; ++j)
#pragma unroll
            for (int l = 0; l < G_::KL; ++l)
                t.k[j][l] = load16_kv(kp + (j * G_::KL + l) * 1024);
    } else {
        // the page is the segment; lane group r/4 reads token group s of its page
        const int P = 1 << c.log2_page;
        const int log2_ns = c.log2_page - G_::LOG2_TPG;
        const int kq = c.lane_r >> 2;
        const int sub = static_cast<int>((T0 + kq * G_::TPG) & (P - 1)) >> G_::LOG2_TPG;
        const uint8_t *kp = c.k_head + static_cast<int64_t>(select4(kq, pg)) * c.page_bytes +
                            ((((c.lane_g << log2_ns) + sub) * 4 + (c.lane_r & 3)) * 16);
#pragma unroll
        for (int j = 0; j < G_::NJ; ++j)
#pragma unroll
            for (int l = 0; l < G_::KL; ++l)
                t.k[j][l] = load16_kv(kp + ((j * G_::KL + l) * 256 << log2_ns));
    }
}

template <bool BF16, int D, bool BIG>
__device__ __forceinline__ void mfma_load_v(MfmaTile<BF16, D> &t, const MfmaCtx<BF16, D> &c,
                                            int64_t T0, const TilePages &pg)
{
    using G_ = Geo<BF16, D>;
    // this lane supplies head dim dt*16 + r over the TPG tokens of group g
    if constexpr (BIG) {
        const int seg = static_cast<int>(T0 & ((int64_t{1} << c.log2_page) - 1)) >> G_::LOG2_TT;
        const uint8_t *vp = c.v_head + static_cast<int64_t>(pg.pid[0]) * c.page_bytes +
                            seg * (G_::TT * D * G_::E) + (c.lane_r * G_::TT + c.lane_g * G_::TPG) * G_::E;
#pragma unroll
        for (int dt = 0; dt < G_::NDT; ++dt)
            t.v[dt] = load16_kv(vp + dt * 16 * G_::TT * G_::E);
    } else {
        const int P = 1 << c.log2_page;
        const int vslot = static_cast<int>((T0 + c.lane_g * G_::TPG) & (P - 1));
        const uint8_t *vp = c.v_head + static_cast<int64_t>(select4(c.lane_g, pg)) * c.page_bytes +
                            ((c.lane_r << c.log2_page) + vslot) * G_::E;
#pragma unroll
        for (int dt = 0; dt < G_::NDT; ++dt)
            t.v[dt] = load16_kv(vp + ((dt * 16 * G_::E) << c.log2_page));
    }
}

template <bool BF16, int D>
struct MfmaState {
    f32x4 o[Geo<BF16, D>::NDT];  // O^T: lane holds head r, dims dt*16 + 4g + 0..3
    float m;                     // running max (log2 units) of head r
    float l;                     // this lane's share of the softmax denominator
};

// S^T = K Q^T for one tile: rows = tokens, columns = the group's heads.
template <bool BF16, int D>
__device__ __forceinline__ void mfma_qk(const MfmaTile<BF16, D> &t,
                                        const bf16x8 (&qop)[Geo<BF16, D>::NC],
                                        f32x4 (&sacc)[Geo<BF16, D>::NJ])
{
    using G_ = Geo<BF16, D>;
#pragma unroll
    for (int j = 0; j < G_::NJ; ++j) {
        sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < G_::NC; ++c) {
            bf16x8 a;
            if constexpr (BF16) {
                a = __builtin_bit_cast(bf16x8, t.k[j][c]);
            } else {
                const u32x4 w = t.k[j][c >> 1];
                a = e4m3x8_to_bf16x8(w[(c & 1) * 2], w[(c & 1) * 2 + 1]);
            }
            sacc[j] = mfma_bf16(a, qop[c], sacc[j]);
        }
    }
}

// Online softmax of one tile's scores, then O^T += V^T P^T (rows = head dims,
// columns = heads).  TAIL masks tokens at or past t1 (only a split's last
// tile can hold such tokens).  DUP (groups of at most 8 heads): column h + 8
// holds a copy of head h (the same query, hence the same scores and softmax
// state), and feeds the low part of P where column h feeds the high part, so
// one MFMA takes both; lo_lane marks the lanes of columns 8..15.
template <bool BF16, int D, bool TAIL, bool DUP>
__device__ __forceinline__ void mfma_softmax_pv(const MfmaTile<BF16, D> &t,
                                                const f32x4 (&sacc)[Geo<BF16, D>::NJ],
                                                MfmaState<BF16, D> &st, float cs, int64_t T0,
                                                int64_t t1, int lane_g, bool lo_lane)
{
    using G_ = Geo<BF16, D>;
    // lane holds the scores of tokens T0 + lane_g*TPG + n, n = 4j + v
    float s[G_::TPG];
#pragma unroll
    for (int j = 0; j < G_::NJ; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            s[4 * j + v] = sacc[j][v];
    int nvalid = G_::TPG;
    if constexpr (TAIL) {
        const int64_t nv = t1 - (T0 + lane_g * G_::TPG);
        nvalid = nv < 0 ? 0 : (nv > G_::TPG ? G_::TPG : static_cast<int>(nv));
#pragma unroll
        for (int n = 0; n < G_::TPG; ++n)
            s[n] = n < nvalid ? s[n] : kNegInf;
    }
    float mx = s[0];
#pragma unroll
    for (int n = 1; n < G_::TPG; ++n)
        mx = __builtin_fmaxf(mx, s[n]);
    mx = __builtin_fmaxf(mx, shfl_xor_f(mx, 16));
    mx = __builtin_fmaxf(mx, shfl_xor_f(mx, 32));
    const float m_new = __builtin_fmaxf(st.m, mx * cs);
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    float pr[G_::TPG];
    float psum = 0.f;
#pragma unroll
    for (int n = 0; n < G_::TPG; ++n) {
        pr[n] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[n], cs, -m_new));
        psum += pr[n];
    }
    st.l = st.l * alpha + psum;
    st.m = m_new;
#pragma unroll
    for (int dt = 0; dt < G_::NDT; ++dt)
        st.o[dt] *= alpha;
    // P enters the P.V MFMAs as a bf16 high part plus a bf16 low part (the
    // rounding error of the high part, itself rounded): together they carry
    // P to about 2^-16 relative, over the whole fp32 exponent range, so that
    // no weight is flushed however peaked the softmax.  V is exact in bf16
    // for both pool types (e4m3 decodes exactly to bf16).
#pragma unroll
    for (int c = 0; c < G_::NPC; ++c) {
        u32x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = pr[c * 8 + 2 * e], b = pr[c * 8 + 2 * e + 1];
            hi[e] = pack_bf16x2(a, b);
            lo[e] = pack_bf16x2(a - bf16_lo(hi[e]), b - bf16_hi(hi[e]));
        }
        u32x4 mine;
        if constexpr (DUP) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                mine[e] = lo_lane ? lo[e] : hi[e];
        }
        const bf16x8 phi = __builtin_bit_cast(bf16x8, DUP ? mine : hi);
        const bf16x8 plo = __builtin_bit_cast(bf16x8, lo);
#pragma unroll
        for (int dt = 0; dt < G_::NDT; ++dt) {
            u32x4 w = t.v[dt];
            bf16x8 a;
            if constexpr (BF16) {
                if constexpr (TAIL)
                    w = keep_bytes(w, nvalid * 2);
                a = __builtin_bit_cast(bf16x8, w);
            } else {
                if constexpr (TAIL)
                    w = keep_bytes(w, nvalid);
                a = e4m3x8_to_bf16x8(w[2 * c], w[2 * c + 1]);
            }
            st.o[dt] = mfma_bf16(a, phi, st.o[dt]);
            if constexpr (!DUP)
                st.o[dt] = mfma_bf16(a, plo, st.o[dt]);
        }
    }
}

// Shared end of both paths: merge the waves' states and write the result.
template <int D>
struct MergeSmem {
    float o[kWaves][16][D + 4];
    float m[kWaves][16];
    float l[kWaves][16];
};

// Where a group's merged rows go: query head h of the group to o + h*stride*D
// and lse[h*stride] (lse may be nullptr).
struct MergeDst {
    float *o;
    float *lse;
    int64_t stride;
};

// final output (one split) or the split's partial rows
template <int D>
__device__ __forceinline__ MergeDst split_dst(const AttnParams &p, int b, int g, int s)
{
    const int64_t bh0 = static_cast<int64_t>(b) * p.num_q_heads + static_cast<int64_t>(g) * p.group;
    if (p.num_splits == 1)
        return MergeDst{p.out + bh0 * D, p.lse != nullptr ? p.lse + bh0 : nullptr, 1};
    const int64_t row0 = bh0 * p.num_splits + s;
    return MergeDst{p.part_o + row0 * D, p.part_lse + row0, p.num_splits};
}

template <int D>
__device__ __forceinline__ void merge_and_write(MergeSmem<D> &sm, int nheads, int state, int bad,
                                                float v_scale, MergeDst dst)
{
    for (int idx = threadIdx.x; idx < nheads * (D / 4); idx += kThreads) {
        const int h = idx / (D / 4);
        const int d4 = (idx % (D / 4)) * 4;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        float lse = kNegInf;
        if (state == 0) {
            float M = kNegInf;
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
                M = __builtin_fmaxf(M, sm.m[w][h]);
            if (M != kNegInf) {
                float Ls = 0.f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    const float mw = sm.m[w][h];
                    const float wt = mw == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mw - M);
                    Ls += wt * sm.l[w][h];
                    const f32x4 ow = *reinterpret_cast<const f32x4 *>(&sm.o[w][h][d4]);
                    o += wt * ow;
                }
                o *= v_scale / Ls;
                lse = (M + __log2f(Ls)) * kLn2;
            }
        }
        if (state == 2 || bad) {
            const float nan = __builtin_nanf("");
            o = f32x4{nan, nan, nan, nan};
            lse = nan;
        }
        const int64_t row = h * dst.stride;
        *reinterpret_cast<f32x4 *>(dst.o + row * D + d4) = o;
        if (d4 == 0 && dst.lse != nullptr)
            dst.lse[row] = lse;
    }
}

// ---------------------------------------------------------------------------
// Balanced partition (num_splits < 0).  For one KV head, the pages of all
// live requests taken in request order form one sequence of T pages; W
// work-groups take consecutive ranges of C = ceil(T / W) pages each, so every
// work-group streams the same bytes however ragged the context lengths are.
// A range may cut a request (and hold several): a request piece lying wholly
// inside one range is the request itself and goes straight to the output;
// any other piece leaves a partial at row b + w of its query head (rows
// [Hq][R], R = B + W - 1).  Pieces (b, w) and (b', w') with b + w == b' + w'
// cannot both exist -- b' > b would make request b' start after b ends while
// range w' ends before w starts -- so a request's partials are the
// consecutive rows b + w_first .. b + w_last, which the balanced combine
// merges.  Work-group 0 of KV head 0 also stores every request's first page
// in the sequence and C, from which the combine finds those rows.
// ---------------------------------------------------------------------------
struct ReqPages {
    int64_t n;  // pages in the sequence (0: aborted, empty or invalid)
    int64_t L;
};

__device__ __forceinline__ ReqPages request_pages(const AttnParams &p, int b)
{
    ReqPages r{0, 0};
    if (p.req_status != nullptr && p.req_status[b] != 0)
        return r;
    const int64_t L = p.context_lens[b];
    if (L <= 0 || L > (static_cast<int64_t>(p.max_pages) << p.log2_page))
        return r;
    r.L = L;
    r.n = (L + (int64_t{1} << p.log2_page) - 1) >> p.log2_page;
    return r;
}

struct BalSmem {
    int64_t wave_total[kWaves];
    int64_t ps0;
    int b0;
};

struct BalRange {
    int64_t lo, hi;  // the work-group's pages of the sequence
    int64_t C;       // pages per work-group
    int64_t ps0;     // sequence offset of request b0's first page
    int b0;          // the request holding page lo (batch if the range is empty)
};

__device__ __forceinline__ int64_t wave_incl_scan(int64_t v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int64_t u = __shfl_up(v, d, 64);
        v += lane >= d ? u : 0;
    }
    return v;
}

// Every work-group scans the request lengths (threads take consecutive runs of
// requests), then finds its range and the request that holds its first page.
__device__ __forceinline__ BalRange bal_range(const AttnParams &p, BalSmem &bs, int w,
                                              bool store_prefix)
{
    const int B = p.batch;
    const int per = (B + kThreads - 1) / kThreads;
    const int first = static_cast<int>(threadIdx.x) * per;
    const int last = first + per < B ? first + per : B;
    int64_t sum = 0;
    for (int b = first; b < last; ++b)
        sum += request_pages(p, b).n;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t incl = wave_incl_scan(sum);
    if (lane == 63)
        bs.wave_total[wave] = incl;
    __syncthreads();
    int64_t before = 0, T = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        before += i < wave ? bs.wave_total[i] : 0;
        T += bs.wave_total[i];
    }
    const int64_t ex = before + incl - sum;  // sequence offset of request `first`
    BalRange r;
    r.C = T > 0 ? (T + p.bal_groups - 1) / p.bal_groups : 1;
    r.lo = static_cast<int64_t>(w) * r.C;
    r.hi = r.lo + r.C < T ? r.lo + r.C : T;
    if (store_prefix) {
        int64_t at = ex;
        for (int b = first; b < last; ++b) {
            p.bal_prefix[b] = at;
            at += request_pages(p, b).n;
        }
        if (threadIdx.x == 0)
            p.bal_prefix[B] = r.C;
    }
    r.b0 = B;
    r.ps0 = T;
    if (r.lo >= r.hi)
        return r;  // uniform: the whole work-group has nothing to do
    // exactly one thread's run of pages [ex, ex + sum) holds page lo
    if (ex <= r.lo && r.lo < ex + sum) {
        int64_t at = ex;
        for (int b = first; b < last; ++b) {
            const int64_t n = request_pages(p, b).n;
            if (r.lo < at + n) {
                bs.b0 = b;
                bs.ps0 = at;
                break;
            }
            at += n;
        }
    }
    __syncthreads();
    r.b0 = bs.b0;
    r.ps0 = bs.ps0;
    return r;
}

// the tokens of the piece of request rq (first page ps in the sequence) that
// falls in range r; page offsets are relative to the request
__device__ __forceinline__ SplitRange piece_range(const AttnParams &p, const BalRange &r,
                                                  int64_t ps, const ReqPages &rq)
{
    const int64_t p0 = (r.lo > ps ? r.lo : ps) - ps;
    const int64_t p1 = (r.hi < ps + rq.n ? r.hi : ps + rq.n) - ps;
    SplitRange s;
    s.t0 = p0 << p.log2_page;
    s.t1 = p1 << p.log2_page;
    if (s.t1 > rq.L)
        s.t1 = rq.L;
    s.p_last = p1 - 1;
    s.state = 0;
    return s;
}

template <int D>
__device__ __forceinline__ MergeDst piece_dst(const AttnParams &p, const BalRange &r, int64_t ps,
                                              const ReqPages &rq, int b, int g, int w)
{
    if (ps >= r.lo && ps + rq.n <= r.hi)  // the whole request
        return split_dst<D>(p, b, g, 0);
    const int64_t R = static_cast<int64_t>(p.batch) + p.bal_groups - 1;
    const int64_t row0 = static_cast<int64_t>(g) * p.group * R + b + w;
    return MergeDst{p.part_o + row0 * D, p.part_lse + row0, R};
}

// A wave's softmax state into sm (row r of the wave's slot holds head r).
template <bool BF16, int D, bool DUP>
__device__ __forceinline__ void mfma_state_to_smem(MfmaState<BF16, D> &st, MergeSmem<D> &sm)
{
    using G_ = Geo<BF16, D>;
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    if constexpr (DUP) {
        // column h + 8 accumulated V times the low part of head h's weights
#pragma unroll
        for (int dt = 0; dt < G_::NDT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                st.o[dt][e] += shfl_xor_f(st.o[dt][e], 8);
    }
    // the four lanes of a head each hold a quarter of its denominator
    float l = st.l + shfl_xor_f(st.l, 16);
    l += shfl_xor_f(l, 32);
    const int r = lane & 15, lg = lane >> 4;
    if (lg == 0) {
        sm.m[wave][r] = st.m;
        sm.l[wave][r] = l;
    }
#pragma unroll
    for (int dt = 0; dt < G_::NDT; ++dt)
        *reinterpret_cast<f32x4 *>(&sm.o[wave][r][dt * 16 + lg * 4]) = st.o[dt];
}

template <bool BF16, int D>
__device__ __forceinline__ void mfma_state_reset(MfmaState<BF16, D> &st)
{
#pragma unroll
    for (int dt = 0; dt < Geo<BF16, D>::NDT; ++dt)
        st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = kNegInf;
    st.l = 0.f;
}

// One wave's softmax state, normalised: lane (r, lg) holds out =
// o * v_scale / l of head r, dims dt*16 + 4*lg .. + 3, and every lane its
// head's lse = ln(sum exp) (the wave-per-split mode, where no other wave
// shares the split).  state / bad as in merge_and_write.
template <bool BF16, int D>
struct WaveRows {
    f32x4 o[Geo<BF16, D>::NDT];
    float lse;
};

template <bool BF16, int D, bool DUP>
__device__ __forceinline__ WaveRows<BF16, D> mfma_state_rows(MfmaState<BF16, D> &st, int state, int bad,
                                                             float v_scale)
{
    using G_ = Geo<BF16, D>;
    if constexpr (DUP) {
#pragma unroll
        for (int dt = 0; dt < G_::NDT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                st.o[dt][e] += shfl_xor_f(st.o[dt][e], 8);
    }
    float l = st.l + shfl_xor_f(st.l, 16);
    l += shfl_xor_f(l, 32);
    float scale = 0.f;
    WaveRows<BF16, D> w;
    w.lse = kNegInf;
    if (state == 0 && st.m != kNegInf) {
        scale = v_scale / l;
        w.lse = (st.m + __log2f(l)) * kLn2;
    }
    const bool nan_rows = state == 2 || bad;
    if (nan_rows)
        w.lse = __builtin_nanf("");
#pragma unroll
    for (int dt = 0; dt < G_::NDT; ++dt)
        w.o[dt] = nan_rows ? f32x4{w.lse, w.lse, w.lse, w.lse} : st.o[dt] * scale;
    return w;
}

template <bool BF16, int D>
__device__ __forceinline__ void store_wave_rows(const WaveRows<BF16, D> &w, int nheads, MergeDst dst)
{
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, lg = lane >> 4;
    if (r < nheads) {
        float *row = dst.o + static_cast<int64_t>(r) * dst.stride * D;
#pragma unroll
        for (int dt = 0; dt < Geo<BF16, D>::NDT; ++dt)
            *reinterpret_cast<f32x4 *>(row + dt * 16 + lg * 4) = w.o[dt];
        if (lg == 0 && dst.lse != nullptr)
            dst.lse[static_cast<int64_t>(r) * dst.stride] = w.lse;
    }
}

// Request b, KV head g over tokens [rng.t0, rng.t1); dst(j) is where split
// j's rows go.
//  * Work-group mode (WAVE false): one split; the four waves take the
//    range's tiles in turn and merge their states through sm at the end.
//  * Wave mode (WAVE true): the calling wave alone streams every tile of the
//    range, which covers nparts <= 2 consecutive splits of part_tiles tiles
//    each (the request's last split may be shorter); at the split boundary
//    it normalises the first split's rows into registers and starts afresh,
//    with the next split's first tile already in flight -- no barrier, no
//    shared memory.  All rows are stored once the range is done: a store in
//    mid-stream would hold up the wave's next loads until memory, busy with
//    every wave's reads, has acknowledged it.
// A page id outside the pool turns the rows written from then on into NaN.
template <bool BF16, int D, bool BIG, bool DUP, bool WAVE, class DstFn>
__device__ __forceinline__ void mfma_range(const AttnParams &p, MergeSmem<D> *sm, int b, int g,
                                           const SplitRange &rng, int nparts, int part_tiles,
                                           float v_scale, DstFn dst)
{
    using G_ = Geo<BF16, D>;
    const int G = p.group;
    const int lane = threadIdx.x & 63;
    const int wave = WAVE ? 0 : uniform(threadIdx.x >> 6);
    constexpr int kStep = WAVE ? 1 : kWaves;  // tiles between a wave's consecutive tiles
    MfmaState<BF16, D> st;
    mfma_state_reset(st);
    int bad = 0;
    int pj = 0;  // next split to write
    WaveRows<BF16, D> held;  // wave mode: the first of two splits' rows
    auto flush = [&]() {
        if constexpr (WAVE) {
            const WaveRows<BF16, D> rows = mfma_state_rows<BF16, D, DUP>(st, rng.state, bad, v_scale);
            if (pj + 1 < nparts) {
                held = rows;
            } else {
                if (nparts == 2)
                    store_wave_rows<BF16, D>(held, G, dst(0));
                store_wave_rows<BF16, D>(rows, G, dst(pj));
            }
        } else {
            mfma_state_to_smem<BF16, D, DUP>(st, *sm);
            const int any_bad = __syncthreads_or(bad);
            merge_and_write<D>(*sm, G, rng.state, any_bad, v_scale, dst(pj));
        }
        mfma_state_reset(st);
        ++pj;
    };

    const int64_t ntok = rng.t1 - rng.t0;
    const int ntiles = rng.state == 0 ? static_cast<int>((ntok + G_::TT - 1) / G_::TT) : 0;
    if (wave < ntiles) {
        MfmaCtx<BF16, D> c;
        const int64_t head_bytes = (int64_t{1} << p.log2_page) * D * G_::E;
        c.page_bytes = head_bytes * p.num_kv_heads;
        c.k_head = p.k_pool + g * head_bytes;
        c.v_head = p.v_pool + g * head_bytes;
        c.log2_page = p.log2_page;
        c.lane_r = lane & 15;
        c.lane_g = lane >> 4;
        // Q operand: head r of the group (with DUP, head r mod 8), head dims
        // [g*D/4, (g+1)*D/4)
        bf16x8 qop[G_::NC];
        {
            const int r = DUP ? (c.lane_r & 7) : c.lane_r;
            const uint16_t *qrow = p.q + (static_cast<int64_t>(b) * p.num_q_heads + g * G + r) * D +
                                   c.lane_g * (D / 4);
#pragma unroll
            for (int cc = 0; cc < G_::NC; ++cc) {
                const u32x4 w = r < G ? load16(qrow + 8 * cc) : u32x4{0u, 0u, 0u, 0u};
                qop[cc] = __builtin_bit_cast(bf16x8, w);
            }
        }
        const float cs = (BF16 ? 1.0f : p.k_scale[g]) * p.sm_scale * kLog2e;
        const page_row_t row = page_row(p, b);
        const int stride = kStep * G_::TT;
        const bool lo_lane = c.lane_r >= 8;
        // wave mode: tiles done, and the count at which the next split opens
        int done = 0;
        int next_cross = WAVE && nparts > 1 ? part_tiles : 0x7FFFFFFF;

        // Staggered pipeline, one tile buffer per wave: the next tile's K is
        // loaded as soon as Q.K^T has consumed this tile's K, and its V as
        // soon as P.V has consumed this tile's V, so each wave always has about
        // one tile (16 KB) in flight without a second register buffer.  Page
        // ids come a tile ahead.  The steady-state loop has no conditional
        // loads (the last tile is peeled), so the compiler waits for exactly
        // the loads each step needs.
        MfmaTile<BF16, D> t;
        f32x4 sacc[G_::NJ];
        int i = wave;
        int64_t T0 = rng.t0 + static_cast<int64_t>(i) * G_::TT;
        {
            const TilePages pg = pages_ok(fetch_pages<BIG>(row, T0, G_::TPG, p.log2_page, rng.p_last),
                                          p.num_pages, bad);
            mfma_load_k<BF16, D, BIG>(t, c, T0, pg);
            mfma_load_v<BF16, D, BIG>(t, c, T0, pg);
        }
        TilePages pgn = fetch_pages<BIG>(row, T0 + stride, G_::TPG, p.log2_page, rng.p_last);
        while (i + kStep < ntiles) {
            const TilePages pn = pages_ok(pgn, p.num_pages, bad);
            mfma_qk(t, qop, sacc);
            // keep each load batch where it is: hoisting it above the
            // computation that frees its registers would need a second buffer
            __builtin_amdgcn_sched_barrier(0);
            mfma_load_k<BF16, D, BIG>(t, c, T0 + stride, pn);
            __builtin_amdgcn_sched_barrier(0);
            mfma_softmax_pv<BF16, D, false, DUP>(t, sacc, st, cs, T0, rng.t1, c.lane_g, lo_lane);
            __builtin_amdgcn_sched_barrier(0);
            mfma_load_v<BF16, D, BIG>(t, c, T0 + stride, pn);
            __builtin_amdgcn_sched_barrier(0);
            pgn = fetch_pages<BIG>(row, T0 + 2 * stride, G_::TPG, p.log2_page, rng.p_last);
            i += kStep;
            T0 += stride;
            if constexpr (WAVE) {
                if (++done == next_cross) {  // the next tile opens the next split
                    flush();
                    next_cross = pj < nparts - 1 ? next_cross + part_tiles : 0x7FFFFFFF;
                }
            }
        }
        mfma_qk(t, qop, sacc);
        if (T0 + G_::TT > rng.t1)
            mfma_softmax_pv<BF16, D, true, DUP>(t, sacc, st, cs, T0, rng.t1, c.lane_g, lo_lane);
        else
            mfma_softmax_pv<BF16, D, false, DUP>(t, sacc, st, cs, T0, rng.t1, c.lane_g, lo_lane);
    }
    while (pj < nparts)  // the last split, and splits past the request's end
        flush();
}

// MI355X deals the work-groups of a launch to its 8 XCDs in turn (block i to
// XCD i mod 8).  This renumbering hands XCD x the x-th contiguous range of
// the launch's n work units instead (ranges of n/8, the first n mod 8 one
// longer), so that the units of one request -- all its KV heads and splits,
// which read the same pages -- share an XCD.  Measured on equal-length
// batches: 64 x 16k e4m3 about 0.6% faster, the bf16 twin and the balanced
// partition about 2%, one query head per KV head 1-3%.  A ragged batch at
// one split per request loses about 2% (the XCDs then carry unequal bytes),
// which the balanced partition is for.  Any n: a bijection of [0, n).
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_unit(int i, int n)
{
    const int x = i % kXcds, k = i / kXcds, q = n / kXcds, r = n % kXcds;
    return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

// Three work-groups per CU where the registers allow it without spilling:
// pages of a whole tile, except the e4m3 kernel that also appends for groups
// of more than 8 heads.
template <bool BF16, int D, bool BIG, bool APPEND, bool DUP>
__global__ __launch_bounds__(kThreads, (BIG && (BF16 || DUP || !APPEND)) ? 3 : 2) void decode_attn_mfma_kernel(
    AttnParams p)
{
    __shared__ MergeSmem<D> sm;

    int idx = xcd_unit(blockIdx.x, gridDim.x);
    const int s = idx % p.num_splits;
    idx /= p.num_splits;
    const int g = idx % p.num_kv_heads;
    const int b = idx / p.num_kv_heads;

    const SplitRange rng = split_range(p, b, s);
    if constexpr (APPEND) {
        const int64_t L = p.context_lens[b];
        if (rng.state == 0 && rng.t0 < rng.t1 && rng.t1 == L)
            append_new_token<BF16, D>(p, b, g, L);
    }
    mfma_range<BF16, D, BIG, DUP, false>(p, &sm, b, g, rng, 1, 0, BF16 ? 1.0f : p.v_scale[g],
                                         [&](int) { return split_dst<D>(p, b, g, s); });
}

// Wave-per-split mode, for launches with at least a split per wave slot of
// the GPU (many splits of long requests): every wave independently takes
// wave_parts consecutive splits of one (request, KV head) -- chunk c of that
// pair -- and writes their partial rows; the combine merges them as usual.
// Splits of a whole number of tiles only.
template <bool BF16, int D, bool BIG, bool DUP>
__global__ __launch_bounds__(kThreads, 2) void decode_attn_mfma_wave_kernel(AttnParams p)
{
    const int64_t gw = static_cast<int64_t>(blockIdx.x) * kWaves + uniform(threadIdx.x >> 6);
    const int64_t nchunks = (p.num_splits + p.wave_parts - 1) / p.wave_parts;
    if (gw >= static_cast<int64_t>(p.batch) * p.num_kv_heads * nchunks)
        return;  // the grid's last work-group may hold idle waves
    const int c = static_cast<int>(gw % nchunks);
    const int g = static_cast<int>((gw / nchunks) % p.num_kv_heads);
    const int b = static_cast<int>(gw / nchunks / p.num_kv_heads);
    const int s0 = c * p.wave_parts;
    const int nparts = p.num_splits - s0 < p.wave_parts ? p.num_splits - s0 : p.wave_parts;
    const SplitRange rng = split_range(p, b, s0, nparts);
    mfma_range<BF16, D, BIG, DUP, true>(p, static_cast<MergeSmem<D> *>(nullptr), b, g, rng, nparts,
                                        p.part_tiles, BF16 ? 1.0f : p.v_scale[g],
                                        [&](int j) { return split_dst<D>(p, b, g, s0 + j); });
}

// Balanced partition: the work-group takes pages [lo, hi) of its KV head's
// concatenated live pages and attends to each request piece in turn.
template <bool BF16, int D, bool BIG, bool APPEND, bool DUP>
__global__ __launch_bounds__(kThreads, 2) void decode_attn_bal_mfma_kernel(AttnParams p)
{
    __shared__ MergeSmem<D> sm;
    __shared__ BalSmem bs;

    const int u = xcd_unit(blockIdx.x, gridDim.x);
    const int g = u % p.num_kv_heads;
    const int w = u / p.num_kv_heads;
    const BalRange r = bal_range(p, bs, w, g == 0 && w == 0);
    int64_t ps = r.ps0;
    for (int b = r.b0; b < p.batch && ps < r.hi; ++b) {
        const ReqPages rq = request_pages(p, b);
        if (rq.n > 0) {
            const SplitRange rng = piece_range(p, r, ps, rq);
            if constexpr (APPEND) {
                if (ps + rq.n <= r.hi)  // the piece ends at the request's last token
                    append_new_token<BF16, D>(p, b, g, rq.L);
            }
            mfma_range<BF16, D, BIG, DUP, false>(p, &sm, b, g, rng, 1, 0, BF16 ? 1.0f : p.v_scale[g],
                                                 [&](int) { return piece_dst<D>(p, r, ps, rq, b, g, w); });
            __syncthreads();  // sm is written again by the next piece
        }
        ps += rq.n;
    }
}

template <bool BF16, int D, bool APPEND, bool DUP>
void launch_mfma_t(const AttnParams &p, dim3 grid, dim3 block, bool bal, hipStream_t stream)
{
    if (p.log2_page >= Geo<BF16, D>::LOG2_TT) {
        if (bal)
            hipLaunchKernelGGL((decode_attn_bal_mfma_kernel<BF16, D, true, APPEND, DUP>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((decode_attn_mfma_kernel<BF16, D, true, APPEND, DUP>), grid, block, 0, stream, p);
    } else {
        if (bal)
            hipLaunchKernelGGL((decode_attn_bal_mfma_kernel<BF16, D, false, APPEND, DUP>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((decode_attn_mfma_kernel<BF16, D, false, APPEND, DUP>), grid, block, 0, stream, p);
    }
}

template <bool BF16, int D, bool APPEND>
hipError_t launch_attn_t(const AttnParams &p, hipStream_t stream)
{
    const bool bal = p.bal_groups > 0;
    const bool wave_mode = p.wave_parts > 0;
    int64_t blocks = bal ? static_cast<int64_t>(p.num_kv_heads) * p.bal_groups
                         : static_cast<int64_t>(p.batch) * p.num_kv_heads * p.num_splits;
    if (wave_mode)
        blocks = (static_cast<int64_t>(p.batch) * p.num_kv_heads *
                      ((p.num_splits + p.wave_parts - 1) / p.wave_parts) + kWaves - 1) / kWaves;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
    if (wave_mode && !APPEND && p.log2_page >= Geo<BF16, D>::LOG2_TT) {
        if (p.group <= 8)
            hipLaunchKernelGGL((decode_attn_mfma_wave_kernel<BF16, D, true, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((decode_attn_mfma_wave_kernel<BF16, D, true, false>), grid, block, 0, stream, p);
    } else if (wave_mode) {
        return hipErrorInvalidValue;  // the host only picks wave mode for whole-page tiles, no append
    } else if (p.group <= 8) {
        launch_mfma_t<BF16, D, APPEND, true>(p, grid, block, bal, stream);
    } else {
        launch_mfma_t<BF16, D, APPEND, false>(p, grid, block, bal, stream);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_attn(bool bf16_pool, int head_dim, const AttnParams &p,
                              hipStream_t stream)
{
    const bool app = p.k_new != nullptr;
    if (bf16_pool) {
        if (head_dim == 64)
            return app ? launch_attn_t<true, 64, true>(p, stream) : launch_attn_t<true, 64, false>(p, stream);
        return app ? launch_attn_t<true, 128, true>(p, stream) : launch_attn_t<true, 128, false>(p, stream);
    }
    if (head_dim == 64)
        return app ? launch_attn_t<false, 64, true>(p, stream) : launch_attn_t<false, 64, false>(p, stream);
    return app ? launch_attn_t<false, 128, true>(p, stream) : launch_attn_t<false, 128, false>(p, stream);
}

}  // namespace pafp8
