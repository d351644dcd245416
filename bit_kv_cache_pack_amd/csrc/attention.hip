// Fused chunk attention over a packed low-bit KV cache plus an unquantized current chunk,
// with the per-score Jensen-bias correction.
//
// Method: "Quantized Keys Steal Attention: Bias Correction for KV-Cache Compression in
// Video Diffusion", abstract: queries of the current chunk attend a quantized cache of
// earlier chunks and their own unquantized chunk; rounding noise on cached keys raises
// their softmax weight on average (exp is convex), which a per-score term computed from
// the keys' step sizes and the query removes to second order. Here that term is
//   beta(i, g) = tau^2/24 * sum_c q_ic^2 step_gc^2
// (half the variance of tau * q . e for e_c uniform on [-step_c/2, step_c/2]),
// subtracted from every logit of a token in K-group g. "KV Cache Quantization for
// Self-Forcing Video Generation", abstract: rebuilding full-precision K/V buffers
// during attention forfeits the memory saved, so dequantized tiles live only in LDS.
// WindowQuant notes ("技術的に面白い点"): windows of one bit-width are stored together;
// each such segment is walked with its own bit-width.
//
// Workgroup: 8 waves, 256 query rows (32 per wave; the rows of one KV head's query heads
// are packed, so GQA decode fills rows) of one (batch, KV head). A workgroup runs a share
// of the (row block, token) work, in pieces cut at row-block ends. A piece's tokens are
// taken in 64-token tiles that never straddle a K-group, listed in bulk in LDS by all
// threads. Pipeline per tile, one barrier per tile:
//   - the packed codes / raw elements of tile i+1 are loaded into registers,
//   - every wave computes tile i out of LDS buffer i%2: S^T = K Q^T with MFMA 32x32x16
//     (lanes own queries, so softmax statistics and the Jensen term are per-lane
//     scalars), online softmax in the log2 domain with rescaling only when a row
//     maximum grows by more than 2^8, O^T += V^T P^T with P in fp16,
//   - all threads dequantize tile i+1 into LDS buffer (i+1)%2.
// LDS rows hold channels in a fixed order: inside each 16-channel block, position
// 4j + k holds channel 4k + j (a 4x4 transpose). Q is loaded in that order, the output
// is written back in channel order. Keys: [token][position] in the element dtype.
// Values: [token][position] in fp16, read into the PV product with the LDS transpose
// load. INT2 values are expanded through a 4-entry table per (token, V group) holding
// the exact dequantized values, indexed with byte permutes; keys and INT4 values use the
// fp16 step/zero directly in mixed-precision fused multiply-adds.
// The Jensen terms of 32 consecutive K-groups are computed at once as a small matrix
// product (step^2 x q^2, each split into bf16 high and low parts, three MFMAs per
// k-step) and read back per group; the isotropic form feeds the group's channel mean of
// step^2 to the same product.
// The serial part of each tile's softmax runs at a raised wave priority, so that the
// other wave of the SIMD issues around it. A piece's output leaves through the wave's
// table in LDS as 16-byte row segments: the final output for a whole row block, otherwise
// unnormalized partials in the workspace, which a combine kernel merges by log-sum-exp.
#include "decode_walk.cuh"
#include "kvq_internal.h"
#include "kvq_quant.cuh"
#include "kvq_tile.cuh"

namespace kvq {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int BM = 32 * kWaves;   // query rows per workgroup
constexpr int TT = 64;    // tokens per tile
// A row of a partial piece: HD int16 mantissas, then m (log2 domain), l and the exponent E
// (the mantissas stand for O 2^(15 - E)) as f32, f32, i32, and a pad word.
template <int HD> struct PieceRow { static constexpr size_t bytes = 2 * HD + 16; };
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescale = 8.0f;  // log2 headroom before the running max is moved

// Row strides (halves) chosen for the 64 LDS banks: key rows 68 dwords apart make the
// 32 MFMA operand reads of a wave conflict-free; value rows 80 (HD 128) or 52 (HD 64)
// dwords apart keep the 4-row transposed reads of each 32-lane half free of conflicts
// (the 16-byte stage writes are, for any stride: each group of 8 lanes writes one row).
template <int HD> struct Geo {
    static constexpr int KROW = HD + 8;
    static constexpr int VROW = HD == 128 ? HD + 32 : HD + 40;
    static constexpr int KBUF = TT * KROW;
    static constexpr int VBUF = TT * VROW;
    static constexpr int BUF = KBUF + VBUF;   // halves per stage buffer
    static constexpr int NBLK = HD / 16;      // 16-channel blocks per row
    static constexpr int UNITS = TT * NBLK;   // (token, block) units per tile, <= kThreads
};

// ---------------------------------------------------------------- tile list
enum : int { TILE_END = 0, TILE_PACKED = 1, TILE_RAW = 2, TILE_CUR = 3, TILE_PTOK = 4 };
// TILE_PTOK: a packed segment with per-token K groups (no K-group table: taken in TT-token
// tiles like raw segments, its keys' step/zero read per token)

// A tile descriptor in four words: kind, segment, flags, Jensen row and bit-width in one.
struct Tile {
    int info;        // kind | segment << 4 | new_group << 8 | batch << 9 | jrow << 10 | bits << 16
    int g, t, len;   // K-group, first token (segment-relative), tokens
    __device__ __forceinline__ int kind() const { return info & 15; }
    __device__ __forceinline__ int seg() const { return (info >> 4) & 15; }
    // first tile of K-group g in this piece
    __device__ __forceinline__ bool new_group() const { return (info >> 8) & 1; }
    // a new block of 32 Jensen terms starts at group g
    __device__ __forceinline__ bool batch() const { return (info >> 9) & 1; }
    // row of group g in its block of 32 Jensen terms
    __device__ __forceinline__ int jrow() const { return (info >> 10) & 31; }
    // the segment's bit-width (16: raw elements)
    __device__ __forceinline__ int bits() const { return info >> 16; }
    // the segment stores the low-rank compensation of its keys
    __device__ __forceinline__ bool comp() const { return (info >> 15) & 1; }
    static __device__ __forceinline__ Tile make(int kind, int seg, int g, int t, int len, int new_group, int jrow,
                                                int bits) {
        return Tile{kind | seg << 4 | new_group << 8 | (new_group && jrow == 0) << 9 | jrow << 10 | bits << 16, g,
                    t, len};
    }
};

__device__ __forceinline__ Tile uniform(Tile t) {
    t.info = __builtin_amdgcn_readfirstlane(t.info);
    t.g = __builtin_amdgcn_readfirstlane(t.g);
    t.t = __builtin_amdgcn_readfirstlane(t.t);
    t.len = __builtin_amdgcn_readfirstlane(t.len);
    return t;
}

// The tiles of a piece are listed in bulk in LDS. A unit is a K-group of a packed segment
// (in the piece) or TT tokens of a raw segment or of the current chunk; every thread takes
// one unit, cuts it into tiles of at most TT tokens that never cross a K-group, and a
// block-wide prefix sum of the tile counts places the tiles in order: segments in order,
// then the current chunk. A list holds at most kListCap tiles; the next one is built when
// the pipeline reaches the end of the current one.
constexpr int kListCap = 512;

struct SegInfo {
    const int32_t *tab;   // K-group table (packed segments)
    int bits, n, ng;      // bit-width (16: raw elements), tokens, K-groups
    int a, e;             // tokens of the piece inside the segment, [a, e)
    int g_lo;             // K-group of token a (packed segments)
    int units;            // units of the segment in the piece
    int ptok, comp;       // per-token K groups; stores the compensation
};

struct TileList {
    Tile t[kListCap];
    SegInfo seg[kMaxSegments + 1];   // the segments, then the current chunk
    int wsum[kWaves];                // prefix-sum scratch: per-wave totals
    int n_tiles;                     // tiles of the list just built
};

// The K-group holding token a: the largest g in [0, ng) whose start is <= a (0 if none),
// for a sorted table. Uniform across the wave; each round reads 64 starts, one per lane,
// and narrows the range 64-fold.
__device__ __forceinline__ int find_group(const int32_t *tab, int ng, int a) {
    const int lane = threadIdx.x % kWave;
    int lo = 0, hi = ng - 1;
    while (lo < hi) {
        const int step = (hi - lo + kWave) / kWave;
        const int g = lo + lane * step;
        const bool ok = g <= hi && group_start(tab, g) <= a;
        const unsigned long long m = __ballot(ok);
        const int k = m ? 63 - __builtin_clzll(m) : 0;
        lo = __builtin_amdgcn_readfirstlane(lo + k * step);
        hi = __builtin_amdgcn_readfirstlane(min(hi, lo + step - 1));
    }
    return lo;
}

// Per piece [tb, te): the range and unit count of each segment, one wave per segment.
// Ends with a barrier.
__device__ __forceinline__ void list_setup(const AttnParams &p, int tb, int te, TileList &L) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    for (int si = wave; si <= p.n_segs; si += kWaves) {
        SegInfo f{nullptr, 16, 0, 0, 0, 0, 0, 0, 0, 0};
        if (si == p.n_segs) {
            const int cb = p.n_total - p.n_cur;
            f.n = p.n_cur;
            f.a = max(tb, cb) - cb;
            f.e = min(te, p.n_total) - cb;
            if (f.e > f.a) f.units = (f.e - f.a + TT - 1) / TT;
        } else {
            const SegmentView &sg = p.segs[si];
            f.tab = sg.kgroup_start;
            f.bits = sg.bits;
            f.n = sg.n_tokens;
            f.ng = sg.bits == 16 ? 0 : sg.n_kgroups;
            f.a = max(tb, sg.token_begin) - sg.token_begin;
            f.e = min(te, sg.token_begin + sg.n_tokens) - sg.token_begin;
            f.ptok = sg.bits != 16 && sg.k_group_channels > 0;
            f.comp = sg.k_comp != nullptr;
            if (f.e > f.a) {
                if (f.bits == 16 || f.ptok) {
                    f.units = (f.e - f.a + TT - 1) / TT;
                } else if (f.ng > 0) {
                    f.g_lo = f.a == 0 ? 0 : find_group(f.tab, f.ng, f.a);
                    const int g_hi = f.e == f.n ? f.ng - 1 : find_group(f.tab, f.ng, f.e - 1);
                    f.units = max(g_hi - f.g_lo + 1, 0);
                }
            }
        }
        if (lane == 0) L.seg[si] = f;
    }
    __syncthreads();
}

// Builds the list of the tiles of units u0, u0 + 1, ... (as many as fit) and returns how
// many units it took; L.n_tiles is its length. All threads call it together; it begins
// by overwriting the list (no wave may still read it) and ends with a barrier.
__device__ __forceinline__ int list_build(const AttnParams &p, TileList &L, int u0, int u_total) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int u = u0 + tid;
    int n = 0, s = 0, g = 0, t0 = 0, t1 = 0, jrow = 0, kind = TILE_END, bits = 16;
    if (u < u_total) {
        int base = 0, i = 0;
        for (int si = 0; si <= p.n_segs; ++si) {
            const int nu = L.seg[si].units;
            if (u >= base && u < base + nu) {
                s = si;
                i = u - base;
            }
            base += nu;
        }
        const SegInfo &f = L.seg[s];
        if (s == p.n_segs || f.bits == 16 || f.ptok) {
            kind = s == p.n_segs ? TILE_CUR : (f.bits == 16 ? TILE_RAW : TILE_PTOK);
            if (kind == TILE_PTOK) bits = f.bits;
            t0 = f.a + TT * i;
            t1 = min(t0 + TT, f.e);
            n = 1;
        } else {
            kind = TILE_PACKED;
            bits = f.bits;
            g = f.g_lo + i;
            // group bounds clamped into the segment: a corrupt table must not send reads outside it
            const int gs = i == 0 ? f.a : min(max(group_start(f.tab, g), 0), f.n);
            const int ge = g + 1 < f.ng ? min(max(group_start(f.tab, g + 1), 0), f.n) : f.n;
            t0 = max(gs, f.a);
            t1 = min(ge, f.e);
            // a valid group has at most 1024 / TT tiles; the cap keeps a corrupt table (one
            // group over a whole segment) from stalling the build
            n = t1 > t0 ? min((t1 - t0 + TT - 1) / TT, kListCap) : 0;
            jrow = i % 32;
        }
    }
    // exclusive prefix sum of n over the block
    int x = n;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == kWave - 1) L.wsum[wave] = x;
    __syncthreads();
    int off = x - n;
    for (int w = 0; w < wave; ++w) off += L.wsum[w];
    // the units that fit are a prefix of the batch
    const bool inc = u < u_total && off + n <= kListCap;
    const int comp_flag = kind == TILE_PACKED && s < p.n_segs && L.seg[s].comp ? 1 << 15 : 0;
    for (int k = 0; inc && k < n; ++k) {
        Tile t = Tile::make(kind, s, g, t0 + TT * k, min(TT, t1 - t0 - TT * k), kind == TILE_PACKED && k == 0,
                            jrow, bits);
        t.info |= comp_flag;
        L.t[off + k] = t;
    }
    const int taken = __syncthreads_count(inc);
    if (taken == 0) {
        if (tid == 0) L.n_tiles = 0;
    } else if (tid == taken - 1) {
        L.n_tiles = off + n;
    }
    __syncthreads();
    return taken;
}

// ---------------------------------------------------------------- prefetch (global -> registers)
// Thread tid owns the unit (token r = tid / NBLK, 16-channel block b = tid % NBLK).
// Raw tiles: w[0..1] = 16 key elements, w[2..3] = 16 value elements. Packed tiles:
// w[0..3] = {step, zero} of the block's 16 key channels, w[4] = a key word pair (x, y) and
// a value word pair (z, w), w[5].x = the token's value {step, zero} for the block.
// With the per-token K columns (AUG), w[6] is the token's source of them: its K step/zero
// row (per-token K groups) or its stored compensation (8 bf16).
template <bool AUG> struct PrefetchT {
    u32x4 w[AUG ? 7 : 6];
};
typedef PrefetchT<false> Prefetch;

// Loads are unconditional, from rows clamped into the tile (staging zeroes rows past it):
// a load under a per-lane condition would have to land before its registers are merged
// with the old contents, which turns every prefetch into a wait for memory.
// The thread index, opaque to the compiler: values derived from it are recomputed where
// they are used instead of being held in registers across the tile loop.
__device__ __forceinline__ int fresh_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

template <int HD, bool AUG>
__device__ __forceinline__ void prefetch_tile(PrefetchT<AUG> &pf, const AttnParams &p, const Tile &tl, size_t bh) {
    typedef Geo<HD> G;
    const int tid = fresh_tid();
    const int r = min(tid / G::NBLK, tl.len - 1), b = tid % G::NBLK;
    if (tl.kind() == TILE_END) return;
    // The same loads for every kind, into the same registers; only their addresses depend
    // on it. w[0..3]: four 16-byte loads (raw keys and values, or the K-group's
    // {step, zero} when it changes). w[4], w[5].x: the packed word pairs and value meta
    // (raw tiles read a harmless copy of their own row).
    const u32x4 *ka = nullptr, *va = nullptr;
    const u32x2 *kp, *vp;
    const uint32_t *vmp;
    bool load4;
    if (tl.kind() == TILE_PACKED || (AUG && tl.kind() == TILE_PTOK)) {
        const SegmentView &sg = p.segs[tl.seg()];
        const int bits = tl.bits();
        const int wpr = HD * bits / 32;   // words per token row
        const size_t row0 = bh * (size_t)sg.capacity + tl.t;
        const uint32_t *kc = reinterpret_cast<const uint32_t *>(sg.k) + row0 * wpr;
        const uint32_t *vc = reinterpret_cast<const uint32_t *>(sg.v) + row0 * wpr;
        // one word pair per thread for either bit-width: INT4 needs words 2b, 2b+1 of the
        // row; INT2 needs word b, and reads the aligned pair around it (still in the row)
        const uint32_t widx = (uint32_t)(r * wpr + (bits == 2 ? (b & ~1) : 2 * b));
        kp = reinterpret_cast<const u32x2 *>(kc + widx);
        vp = reinterpret_cast<const u32x2 *>(vc + widx);
        vmp = sg.v_meta + row0 * (HD / 32) + (uint32_t)(r * (HD / 32) + b / 2);
        if constexpr (AUG) {
            if (tl.kind() == TILE_PTOK) {
                // per-token K groups: the {step, zero} of the thread's block (one group: the
                // group width is at least 32 channels), and the token's whole row of them for
                // the Jensen columns
                const int ng = HD / sg.k_group_channels;
                const uint32_t *krow = sg.k_meta + (row0 + r) * ng;
                pf.w[0].x = krow[(16 * b) / sg.k_group_channels];
                if (ng == 4) {
                    pf.w[6] = *reinterpret_cast<const u32x4 *>(krow);
                } else if (ng == 2) {
                    const u32x2 m = *reinterpret_cast<const u32x2 *>(krow);
                    pf.w[6] = u32x4{m.x, m.y, 0u, 0u};
                } else {
                    pf.w[6] = u32x4{krow[0], 0u, 0u, 0u};
                }
                load4 = false;
            } else {
                if (tl.comp()) pf.w[6] = *reinterpret_cast<const u32x4 *>(sg.k_comp + (row0 + r) * 8);
                ka = reinterpret_cast<const u32x4 *>(sg.k_meta + (bh * sg.kgroup_capacity + tl.g) * HD) + 4 * b;
                va = ka + 2;
                load4 = tl.new_group();
            }
        } else {
            // the {step, zero} of the thread's 16 channels change only with the K-group (a thread
            // keeps its channel block from tile to tile; raw tiles are followed by a new group)
            ka = reinterpret_cast<const u32x4 *>(sg.k_meta + (bh * sg.kgroup_capacity + tl.g) * HD) + 4 * b;
            va = ka + 2;
            load4 = tl.new_group();
        }
    } else {
        const uint16_t *kb, *vb;
        if (tl.kind() == TILE_RAW) {
            const SegmentView &sg = p.segs[tl.seg()];
            const size_t row0 = bh * (size_t)sg.capacity + tl.t;
            kb = reinterpret_cast<const uint16_t *>(sg.k) + row0 * HD;
            vb = reinterpret_cast<const uint16_t *>(sg.v) + row0 * HD;
        } else {
            const size_t row0 = bh * (size_t)p.n_cur + tl.t;
            kb = reinterpret_cast<const uint16_t *>(p.k_cur) + row0 * HD;
            vb = reinterpret_cast<const uint16_t *>(p.v_cur) + row0 * HD;
        }
        ka = reinterpret_cast<const u32x4 *>(kb) + (uint32_t)(r * (HD / 8) + 2 * b);
        va = reinterpret_cast<const u32x4 *>(vb) + (uint32_t)(r * (HD / 8) + 2 * b);
        kp = reinterpret_cast<const u32x2 *>(ka);
        vp = reinterpret_cast<const u32x2 *>(va);
        vmp = reinterpret_cast<const uint32_t *>(ka);
        load4 = true;
    }
    if (load4) {
        pf.w[0] = ka[0];
        pf.w[1] = ka[1];
        pf.w[2] = va[0];
        pf.w[3] = va[1];
    }
    const u32x2 k2 = *kp, v2 = *vp;
    pf.w[4] = u32x4{k2.x, k2.y, v2.x, v2.y};
    pf.w[5].x = *vmp;
}

// ---------------------------------------------------------------- staging (registers -> LDS)
enum : int { STAGE_NONE = 0, STAGE_INT2 = 1, STAGE_INT4 = 2, STAGE_RAW = 3, STAGE_INT2T = 4, STAGE_INT4T = 5 };

__device__ __forceinline__ int stage_kind(const Tile &tl) {
    if (tl.kind() == TILE_END) return STAGE_NONE;
    if (tl.kind() == TILE_PTOK) return tl.bits() == 2 ? STAGE_INT2T : STAGE_INT4T;
    if (tl.kind() != TILE_PACKED) return STAGE_RAW;
    return tl.bits() == 2 ? STAGE_INT2 : STAGE_INT4;
}

// The thread's unit of a prefetched tile, dequantized: 16 keys (element dtype) and 16
// values (fp16), position order. Rows past the tile's end hold a copy of its last row
// (the loads are clamped); their scores are masked, so they add nothing.
template <int SK, bool BF16, bool AUG>
__device__ __forceinline__ void dequant_unit(const PrefetchT<AUG> &pf, int b, uint32_t (&ko)[8], uint32_t (&vo)[8]) {
    typedef Elem<BF16> E;
    if constexpr (SK == STAGE_RAW) {
        const uint32_t kd8[8] = {pf.w[0].x, pf.w[0].y, pf.w[0].z, pf.w[0].w, pf.w[1].x, pf.w[1].y, pf.w[1].z, pf.w[1].w};
        const uint32_t vd8[8] = {E::raw_to_f16(pf.w[2].x), E::raw_to_f16(pf.w[2].y), E::raw_to_f16(pf.w[2].z),
                                 E::raw_to_f16(pf.w[2].w), E::raw_to_f16(pf.w[3].x), E::raw_to_f16(pf.w[3].y),
                                 E::raw_to_f16(pf.w[3].z), E::raw_to_f16(pf.w[3].w)};
        to_positions(kd8, ko);
        to_positions(vd8, vo);
    } else {
        uint32_t km[16];  // {step, zero} of the block's channels, channel order
        if constexpr (SK == STAGE_INT2T || SK == STAGE_INT4T) {
#pragma unroll
            for (int i = 0; i < 16; ++i) km[i] = pf.w[0].x;   // per-token K group: one for the block
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                km[4 * i] = pf.w[i].x; km[4 * i + 1] = pf.w[i].y; km[4 * i + 2] = pf.w[i].z; km[4 * i + 3] = pf.w[i].w;
            }
        }
        const u32x4 c = pf.w[4];   // key word pair, value word pair
        const uint32_t vmeta = pf.w[5].x;
        if constexpr (SK == STAGE_INT2 || SK == STAGE_INT2T) {
            const bool odd = b & 1;
            k2_block<BF16>(odd ? c.y : c.x, km, ko);
            uint32_t tlo, thi;
            v_int2_table<BF16>(vmeta, tlo, thi);
            v_int2_block(odd ? c.w : c.z, tlo, thi, vo);
        } else {
            k4_block<BF16>(c.x, c.y, km, ko);
            v4_block<BF16>(c.z, c.w, vmeta, vo);
        }
    }
}

template <int HD>
__device__ __forceinline__ void write_unit(uint16_t *buf, const uint32_t (&ko)[8], const uint32_t (&vo)[8]) {
    typedef Geo<HD> G;
    const int tid = threadIdx.x;
    const int r = tid / G::NBLK, b = tid % G::NBLK;
    if (G::UNITS >= kThreads || tid < G::UNITS) {
        u32x4 *kd = reinterpret_cast<u32x4 *>(buf + r * G::KROW + 16 * b);
        u32x4 *vd = reinterpret_cast<u32x4 *>(buf + G::KBUF + r * G::VROW + 16 * b);
        kd[0] = u32x4{ko[0], ko[1], ko[2], ko[3]};
        kd[1] = u32x4{ko[4], ko[5], ko[6], ko[7]};
        vd[0] = u32x4{vo[0], vo[1], vo[2], vo[3]};
        vd[1] = u32x4{vo[4], vo[5], vo[6], vo[7]};
    }
}

// Per-token K columns (AUG): 16 bf16 per token, row stride AROW halves. Per-token K groups
// put the squares of the token's group steps there, split into high and low bf16 parts:
// [hi_0..3 | lo_0..3 | hi_0..3 | 0], against the query's [k q2hi_0..3 | k q2hi_0..3 |
// k q2lo_0..3 | 0] (k = -tau / 24), so that one more MFMA k-step adds -beta_t / tau to each
// score; the compensation puts the token's stored c there twice, [c_0..7 | c_0..7], against
// [(U^T q)hi_0..7 | (U^T q)lo_0..7]. Other tiles write zeros. Mode 0 zeros, 1 per-token K
// groups, 2 compensation.
constexpr int AROW = 24;
enum : int { AUG_ZERO = 0, AUG_TOKEN = 1, AUG_COMP = 2 };

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) { return pack_bf16x2(lo, hi); }

template <int HD, bool AUG>
__device__ __forceinline__ void write_aug(uint16_t *abuf, const PrefetchT<AUG> &pf, int mode) {
    if constexpr (AUG) {
        typedef Geo<HD> G;
        const int tid = threadIdx.x;
        if (tid % G::NBLK != 0 || tid / G::NBLK >= TT) return;
        u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
        if (mode == AUG_TOKEN) {
            float d[4], dh[4], dl[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float st = f16_bits_to_f32(pf.w[6][g] & 0xffffu);
                d[g] = st * st;
                dh[g] = (float)(__bf16)d[g];
                dl[g] = d[g] - dh[g];
            }
            lo = u32x4{bf16_pair(dh[0], dh[1]), bf16_pair(dh[2], dh[3]), bf16_pair(dl[0], dl[1]), bf16_pair(dl[2], dl[3])};
            hi = u32x4{lo.x, lo.y, 0u, 0u};
        } else if (mode == AUG_COMP) {
            lo = pf.w[6];
            hi = pf.w[6];
        }
        u32x4 *dst = reinterpret_cast<u32x4 *>(abuf + (tid / G::NBLK) * AROW);
        dst[0] = lo;
        dst[1] = hi;
    }
}

template <int HD, bool BF16, int SK, bool AUG>
__device__ __forceinline__ void stage_only(uint16_t *buf, uint16_t *abuf, const PrefetchT<AUG> &pf, int amode) {
    uint32_t ko[8], vo[8];
    dequant_unit<SK, BF16, AUG>(pf, threadIdx.x % Geo<HD>::NBLK, ko, vo);
    write_unit<HD>(buf, ko, vo);
    write_aug<HD, AUG>(abuf, pf, amode);
}

template <int HD, bool BF16, bool AUG>
__device__ __forceinline__ void stage_tile(uint16_t *buf, uint16_t *abuf, const PrefetchT<AUG> &pf, int sk,
                                           int amode) {
    if (sk == STAGE_INT2) stage_only<HD, BF16, STAGE_INT2, AUG>(buf, abuf, pf, amode);
    else if (sk == STAGE_INT4) stage_only<HD, BF16, STAGE_INT4, AUG>(buf, abuf, pf, amode);
    else if (sk == STAGE_RAW) stage_only<HD, BF16, STAGE_RAW, AUG>(buf, abuf, pf, amode);
    else if constexpr (AUG) {
        if (sk == STAGE_INT2T) stage_only<HD, BF16, STAGE_INT2T, AUG>(buf, abuf, pf, amode);
        else if (sk == STAGE_INT4T) stage_only<HD, BF16, STAGE_INT4T, AUG>(buf, abuf, pf, amode);
    }
}

// ---------------------------------------------------------------- per-wave state and compute
template <int HD, bool BF16> struct Ctx {
    typedef Elem<BF16> E;
    typedef typename E::vec vec;
    static constexpr int KS = HD / 16;   // k-steps of the QK product
    static constexpr int DB = HD / 32;   // 32-position blocks of the output
    vec q[KS];        // this lane's query at positions 16 ks + 8 hh + i
    f32x16 o[DB];     // O^T accumulators, rows = positions
    float *btab;      // LDS [32 K-groups][32 queries]: Jensen sums of the current block of groups
    float m, l;       // running max (log2 domain) and this lane's partial row sum
    float beta;       // Jensen term of the current group, log2 domain
    bf16x8 qa;        // B operand of the per-token K columns (k-slots 8 hh .. 8 hh + 7), AUG only
};

// Jensen sums of K-groups g0 .. g0+31 of a segment for the wave's 32 queries:
// sum over positions of step^2 * q^2, as three bf16 MFMAs on high/low splits. In the
// isotropic form every position's step^2 is the group's mean over its channels, which
// makes the sum |q|^2 * mean_c step_c^2.
template <int HD, bool BF16>
__device__ __forceinline__ void beta_block(Ctx<HD, BF16> &cx, const SegmentView &sg, size_t bh, int g0, bool iso) {
    typedef Ctx<HD, BF16> C;
    const int lane = threadIdx.x % kWave, r32 = lane % 32, hh = lane / 32;
    const int g = g0 + r32;
    const bool ok = g < sg.n_kgroups;
    // this lane's channels in block ks: 4k + 2hh (elements i = k) and 4k + 2hh + 1 (i = 4 + k)
    const uint32_t *km = sg.k_meta + (bh * sg.kgroup_capacity + (ok ? g : 0)) * HD + 2 * hh;
    float mean = 0.f;
    if (iso) {
        // this lane's half of the group's channels, then the other half (lane ^ 32)
        float sum = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const u32x2 v = ok ? *reinterpret_cast<const u32x2 *>(km + 16 * ks + 4 * k) : u32x2{0u, 0u};
                const float s0 = f16_bits_to_f32(v.x & 0xffffu), s1 = f16_bits_to_f32(v.y & 0xffffu);
                sum = __builtin_fmaf(s0, s0, sum);
                sum = __builtin_fmaf(s1, s1, sum);
            }
        mean = (sum + other_half(sum)) * (1.0f / HD);
    }
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        uint32_t m[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const u32x2 v = ok ? *reinterpret_cast<const u32x2 *>(km + 16 * ks + 4 * k) : u32x2{0u, 0u};
            m[k] = v.x;
            m[4 + k] = v.y;
        }
        // opaque: the squares below are derived here, not hoisted out of the tile loop (the
        // queries do not change within a piece) and kept in scratch memory
        u32x4 qw = __builtin_bit_cast(u32x4, cx.q[ks]);
        asm volatile("" : "+v"(qw));
        bf16x8 ah, al, bh8, bl8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // position 16 ks + 8 hh + i holds channel 4 (i % 4) + 2 hh + i / 4 of the block
            const float st = f16_bits_to_f32(m[i] & 0xffffu);
            const float s2 = iso ? mean : st * st;
            const __bf16 s2h = (__bf16)s2;
            ah[i] = s2h;
            al[i] = (__bf16)(s2 - (float)s2h);
            const uint32_t qb = (qw[i / 2] >> (16 * (i % 2))) & 0xffffu;
            const float qv = C::E::val(qb);
            const float q2 = qv * qv;
            const __bf16 q2h = (__bf16)q2;
            bh8[i] = q2h;
            bl8[i] = (__bf16)(q2 - (float)q2h);
        }
        acc = mfma32_bf16(ah, bh8, acc);
        acc = mfma32_bf16(ah, bl8, acc);
        acc = mfma32_bf16(al, bh8, acc);
    }
    // C layout: acc[j] is group 8 (j / 4) + 4 hh + j % 4 of the block, for query r32. The
    // wave alone writes and reads its table, and one wave's LDS operations complete in order.
#pragma unroll
    for (int j = 0; j < 16; ++j) cx.btab[(8 * (j / 4) + 4 * hh + (j % 4)) * 32 + r32] = acc[j];
}

// The all-orders Jensen terms of K-groups g0 .. g0+31 for the wave's 32 queries, log2
// domain: beta = sum over channels of G(a), G(a) = log2(sinh(a) / a), a = (tau / 2) |q_c|
// step_c. With qm_c = (tau / 2) max over the wave's rows of |q_c| (the wave's table, see
// exact_qmax), a^2 = u_q u_d with u_q = (q_c / max|q_c|)^2 <= 1 and u_d = (qm_c step_c)^2.
// Where u_d <= 1, so a <= 1 for every row, G is its Taylor series in a^2 to the fifth
// term (the sixth is below 2.7e-7), and the sum over channels of each term is a matrix
// product over channels of u_q^k and u_d^k, as beta_block's (bf16 high and low parts for the
// first two terms, high parts for the rest, each below 5.1e-4). The (group, channel)
// pairs with u_d > 1, few (channels with outlying steps), are left out of the products and
// evaluated directly for every row afterwards (exact_fallback).
constexpr float kExactC[5] = {0.24044917f, -8.0149723e-3f, 5.0888713e-4f, -3.8166535e-5f, 3.0841645e-6f};
// log2(e) times 1/6, -1/180, 1/2835, -1/37800, 1/467775

// x = qm_c step_c beyond the series' range: the one test both beta_block_poly and
// exact_fallback take.
__device__ __forceinline__ bool outside_series(float x) { return x > 1.0f; }

template <int HD, bool BF16>
__device__ __forceinline__ void beta_block_poly(Ctx<HD, BF16> &cx, const SegmentView &sg, size_t bh, int g0,
                                                const float *qmt, uint32_t (&bigmask)[2]) {
    typedef Ctx<HD, BF16> C;
    const int lane = threadIdx.x % kWave, r32 = lane % 32, hh = lane / 32;
    const int g = g0 + r32;
    const bool ok = g < sg.n_kgroups;
    // this lane's channels in block ks: 4k + 2hh (elements i = k) and 4k + 2hh + 1 (i = 4 + k)
    const uint32_t *km = sg.k_meta + (bh * sg.kgroup_capacity + (ok ? g : 0)) * HD + 2 * hh;
    f32x16 acc = {};
    uint32_t big[2] = {0u, 0u};   // this lane's group: bit 8 ks + i of its positions
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        float ud[8], uq[8];
        {
            uint32_t m[8];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const u32x2 v = ok ? *reinterpret_cast<const u32x2 *>(km + 16 * ks + 4 * kk) : u32x2{0u, 0u};
                m[kk] = v.x;
                m[4 + kk] = v.y;
            }
            // opaque: the query side is derived here, not hoisted out of the tile loop
            u32x4 qw = __builtin_bit_cast(u32x4, cx.q[ks]);
            asm volatile("" : "+v"(qw));
            const f32x4 *qv4 = reinterpret_cast<const f32x4 *>(qmt + 16 * ks + 8 * hh);
            const f32x4 *rv4 = reinterpret_cast<const f32x4 *>(qmt + HD + 16 * ks + 8 * hh);
            const f32x4 qa = qv4[0], qb = qv4[1], ra = rv4[0], rb = rv4[1];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float qmi = i < 4 ? qa[i] : qb[i - 4], rqi = i < 4 ? ra[i] : rb[i - 4];
                const float x = f16_bits_to_f32(m[i] & 0xffffu) * qmi;
                const bool bg = outside_series(x);
                big[(8 * ks + i) / 32] |= (bg ? 1u : 0u) << ((8 * ks + i) % 32);
                ud[i] = bg ? 0.f : x * x;
                const float t = C::E::val((qw[i / 2] >> (16 * (i % 2))) & 0xffffu) * rqi;
                uq[i] = t * t;
            }
        }
        // terms in increasing order, each power from the previous one
        float pd[8], pq[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            pd[i] = ud[i];
            pq[i] = uq[i];
        }
#pragma unroll
        for (int k = 0; k < 5; ++k) {
            bf16x8 ah, bh8, al, bl8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float qv = kExactC[k] * pq[i];
                const __bf16 dh = (__bf16)pd[i], qh = (__bf16)qv;
                ah[i] = dh;
                bh8[i] = qh;
                if (k < 2) {
                    al[i] = (__bf16)(pd[i] - (float)dh);
                    bl8[i] = (__bf16)(qv - (float)qh);
                }
                if (k < 4) {
                    pd[i] *= ud[i];
                    pq[i] *= uq[i];
                }
            }
            acc = mfma32_bf16(ah, bh8, acc);
            if (k < 2) {
                acc = mfma32_bf16(ah, bl8, acc);
                acc = mfma32_bf16(al, bh8, acc);
            }
        }
    }
    // C layout: acc[j] is group 8 (j / 4) + 4 hh + j % 4 of the block, for query r32. The
    // wave alone writes and reads its table, and one wave's LDS operations complete in order.
#pragma unroll
    for (int j = 0; j < 16; ++j) cx.btab[(8 * (j / 4) + 4 * hh + (j % 4)) * 32 + r32] = acc[j];
    // the positions outlying in any group of the block, for the whole wave
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        uint32_t v = big[w];
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) v |= __shfl_xor(v, o);
        bigmask[w] = v;   // lanes of half hh: the positions 16 ks + 8 hh + i, bit 8 ks + i
    }
}

// The (group, channel) pairs beta_block_poly left out: G(a) of every row of the wave, added
// to its table. Positions with a bit in either half's mask are walked one at a time (uniform);
// each lane takes its row's query element at the position (from the half holding it), and
// each group's step is read once per position.
template <int HD, bool BF16>
__device__ __forceinline__ void exact_fallback(Ctx<HD, BF16> &cx, const SegmentView &sg, size_t bh, int g0,
                                               const float *qmt, const uint32_t (&bigmask)[2], float half_scale) {
    typedef Ctx<HD, BF16> C;
    const int lane = threadIdx.x % kWave, r32 = lane % 32, hh = lane / 32;
    const int ng = min(32, sg.n_kgroups - g0);
    for (int h2 = 0; h2 < 2; ++h2) {
        for (int w = 0; w < 2; ++w) {
            // the mask of half h2 (lanes 32 h2 .. 32 h2 + 31 hold it)
            uint32_t mask = __builtin_amdgcn_readlane(bigmask[w], 32 * h2);
            while (mask != 0u) {
                const int bit = __builtin_ctz(mask);
                mask &= mask - 1u;
                const int pidx = 32 * w + bit;          // 8 ks + i
                const int ks = pidx / 8, i = pidx % 8;
                const int pos = 16 * ks + 8 * h2 + i;   // position in the row
                const int ch = 16 * ks + 4 * (i % 4) + 2 * h2 + i / 4;
                // this lane's query element at (ks, i) of its own half; the row's value at the
                // position comes from the half h2 lane of the same row
                // static walk over the lane's elements: no register array indexed at run time
                uint32_t h16 = 0u;
#pragma unroll
                for (int k = 0; k < C::KS; ++k) {
                    const u32x4 qw = __builtin_bit_cast(u32x4, cx.q[k]);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (8 * k + e == pidx) h16 = (qw[e / 2] >> (16 * (e % 2))) & 0xffffu;
                }
                const float mine = C::E::val(h16);
                const float there = other_half(mine);
                const float qv = hh == h2 ? mine : there;
                const float qmi = qmt[pos];
                const float aq = half_scale * __builtin_fabsf(qv);
                for (int gi = 0; gi < ng; ++gi) {
                    const uint32_t mt = group_start(reinterpret_cast<const int32_t *>(sg.k_meta) +
                                                        (bh * sg.kgroup_capacity + g0 + gi) * HD, ch);
                    const float st = f16_bits_to_f32(mt & 0xffffu);
                    if (outside_series(st * qmi)) {   // the pair beta_block_poly left out
                        const float v = log2_sinhc(aq * st);
                        if (hh == 0) cx.btab[gi * 32 + r32] += v;
                    }
                }
            }
        }
    }
}

// qm of the wave's table: (tau / 2) max over the wave's 32 rows of |q| per position, then
// its reciprocal (0 for a zero column), [HD] each.
template <int HD, bool BF16>
__device__ __forceinline__ void exact_qmax(const Ctx<HD, BF16> &cx, float half_scale, float *qmt) {
    typedef Ctx<HD, BF16> C;
    const int lane = threadIdx.x % kWave, r32 = lane % 32, hh = lane / 32;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        const u32x4 qw = __builtin_bit_cast(u32x4, cx.q[ks]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float v = __builtin_fabsf(C::E::val((qw[i / 2] >> (16 * (i % 2))) & 0xffffu));
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
            if (r32 == 0) {
                const float qm = half_scale * v;
                qmt[16 * ks + 8 * hh + i] = qm;
                qmt[HD + 16 * ks + 8 * hh + i] = qm > 0.f ? 1.0f / v : 0.f;
            }
        }
    }
}

// The Jensen sum of group row rr (0..31) of the current block for this lane's query.
template <int HD, bool BF16>
__device__ __forceinline__ float beta_of(const Ctx<HD, BF16> &cx, int rr) {
    return cx.btab[rr * 32 + (fresh_tid() % 32)];
}

// Scheduling masks of the instruction-group barriers
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedDsRead = 0x100, kSchedDsWrite = 0x200;

// One of 8 slices of the dequantization of the thread's unit (k = 0..7: keys in 0..3,
// values in 4..7), so that it can be spread between matrix products. ko / vo complete after
// slices 3 / 7; tab carries the INT2 value table from slice 4 on.
template <int SK, bool BF16, bool AUG>
__device__ __forceinline__ void dequant_slice(const PrefetchT<AUG> &pf, int b, int k, uint32_t (&ko)[8],
                                              uint32_t (&vo)[8], uint32_t (&tab)[2]) {
    typedef Elem<BF16> E;
    if constexpr (SK == STAGE_RAW) {
        // keys: 16-bit elements to position order; values: to fp16 as well
        if (k == 0) {
            const uint32_t kd8[8] = {pf.w[0].x, pf.w[0].y, pf.w[0].z, pf.w[0].w,
                                     pf.w[1].x, pf.w[1].y, pf.w[1].z, pf.w[1].w};
            to_positions(kd8, ko);
        } else if (k == 4) {
            const uint32_t vd8[8] = {E::raw_to_f16(pf.w[2].x), E::raw_to_f16(pf.w[2].y), E::raw_to_f16(pf.w[2].z),
                                     E::raw_to_f16(pf.w[2].w), E::raw_to_f16(pf.w[3].x), E::raw_to_f16(pf.w[3].y),
                                     E::raw_to_f16(pf.w[3].z), E::raw_to_f16(pf.w[3].w)};
            to_positions(vd8, vo);
        }
    } else if constexpr (SK == STAGE_INT2 || SK == STAGE_INT4 || SK == STAGE_INT2T || SK == STAGE_INT4T) {
        constexpr bool TOK = SK == STAGE_INT2T || SK == STAGE_INT4T;   // per-token K group: one step/zero
        const uint32_t km[16] = {pf.w[0].x, TOK ? pf.w[0].x : pf.w[0].y, TOK ? pf.w[0].x : pf.w[0].z,
                                 TOK ? pf.w[0].x : pf.w[0].w, TOK ? pf.w[0].x : pf.w[1].x, TOK ? pf.w[0].x : pf.w[1].y,
                                 TOK ? pf.w[0].x : pf.w[1].z, TOK ? pf.w[0].x : pf.w[1].w, TOK ? pf.w[0].x : pf.w[2].x,
                                 TOK ? pf.w[0].x : pf.w[2].y, TOK ? pf.w[0].x : pf.w[2].z, TOK ? pf.w[0].x : pf.w[2].w,
                                 TOK ? pf.w[0].x : pf.w[3].x, TOK ? pf.w[0].x : pf.w[3].y, TOK ? pf.w[0].x : pf.w[3].z,
                                 TOK ? pf.w[0].x : pf.w[3].w};
        const u32x4 c = pf.w[4];   // key word pair, value word pair
        if constexpr (SK == STAGE_INT2 || SK == STAGE_INT2T) {
            const bool odd = b & 1;
            if (k < 4) {
                k2_step<BF16>(odd ? c.y : c.x, km, k, ko);
            } else {
                if (k == 4) v_int2_table<BF16>(pf.w[5].x, tab[0], tab[1]);
                v_int2_step(odd ? c.w : c.z, tab[0], tab[1], k - 4, vo);
            }
        } else {
            if (k == 0 || k == 2) k4_step<BF16>(c.x, c.y, km, k / 2, ko);
            else if (k == 4 || k == 6) v4_step<BF16>(c.z, c.w, pf.w[5].x, (k - 4) / 2, vo);
        }
    }
}

template <int HD>
__device__ __forceinline__ void write_keys(uint16_t *buf, const uint32_t (&ko)[8]) {
    typedef Geo<HD> G;
    const int tid = threadIdx.x;
    if (G::UNITS >= kThreads || tid < G::UNITS) {
        u32x4 *kd = reinterpret_cast<u32x4 *>(buf + (tid / G::NBLK) * G::KROW + 16 * (tid % G::NBLK));
        kd[0] = u32x4{ko[0], ko[1], ko[2], ko[3]};
        kd[1] = u32x4{ko[4], ko[5], ko[6], ko[7]};
    }
}
template <int HD>
__device__ __forceinline__ void write_values(uint16_t *buf, const uint32_t (&vo)[8]) {
    typedef Geo<HD> G;
    const int tid = threadIdx.x;
    if (G::UNITS >= kThreads || tid < G::UNITS) {
        u32x4 *vd = reinterpret_cast<u32x4 *>(buf + G::KBUF + (tid / G::NBLK) * G::VROW + 16 * (tid % G::NBLK));
        vd[0] = u32x4{vo[0], vo[1], vo[2], vo[3]};
        vd[1] = u32x4{vo[4], vo[5], vo[6], vo[7]};
    }
}

// S^T = K Q^T for the tile in LDS buffer kl (two 32-token halves, s[rb]), while the
// thread's unit of the next tile is dequantized into LDS buffer nbuf. A wave issues in
// order, so the dequantization is written between the products: the matrix core works
// through each product while the vector unit converts. Operand reads run LEAD products
// ahead through a ring of registers.
template <int HD, bool BF16, int SK, bool AUG>
__device__ __forceinline__ void qk_stage(const Ctx<HD, BF16> &cx, const uint16_t *kl, uint16_t *nbuf,
                                         const uint16_t *acur, uint16_t *anext, const PrefetchT<AUG> &pf,
                                         f32x16 (&s)[2], int amode) {
    typedef Ctx<HD, BF16> C;
    typedef typename C::vec vec;
    typedef Geo<HD> G;
    constexpr int NP = 2 * C::KS;    // products
    constexpr int LEAD = 2;          // operand reads ahead of their product
    constexpr int EVERY = NP / 8;    // products per dequantization slice
    const int lane = threadIdx.x % kWave, r32 = lane % 32, hh = lane / 32;
    const int b = threadIdx.x % G::NBLK;
    const uint16_t *kr = kl + r32 * G::KROW + 8 * hh;
    uint32_t ko[8], vo[8], tab[2];
    vec ka[LEAD + 1];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < LEAD; ++i) ka[i] = *reinterpret_cast<const vec *>(kr + 32 * (i / C::KS) * G::KROW + 16 * (i % C::KS));
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        if (i + LEAD < NP) {
            const int n = i + LEAD;
            ka[n % (LEAD + 1)] = *reinterpret_cast<const vec *>(kr + 32 * (n / C::KS) * G::KROW + 16 * (n % C::KS));
        }
        s[i / C::KS] = C::E::mma(ka[i % (LEAD + 1)], cx.q[i % C::KS], s[i / C::KS]);
        if (i % EVERY == 0) {
            const int k = i / EVERY;
            dequant_slice<SK, BF16, AUG>(pf, b, k, ko, vo, tab);
            if (SK != STAGE_NONE && k == 3) write_keys<HD>(nbuf, ko);
            if (SK != STAGE_NONE && k == 7) write_values<HD>(nbuf, vo);
        }
    }
    // keep the written order: per product, its operand read ahead, the product, a slice
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, LEAD, 0);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        if (i + LEAD < NP) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 6, 0);
        if (i == NP / 2 - 1 || i == NP - 1) __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (AUG) {
        // the per-token K columns: one more k-step per 32-token half, bf16 whatever the
        // element dtype; and the next tile's columns into the other buffer
        if (SK != STAGE_NONE) write_aug<HD, AUG>(anext, pf, amode);
        const uint16_t *ar = acur + r32 * AROW + 8 * hh;
        const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(ar);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(ar + 32 * AROW);
        s[0] = mfma32_bf16(a0, cx.qa, s[0]);
        s[1] = mfma32_bf16(a1, cx.qa, s[1]);
    }
}

// Two of the 8 probabilities of the 16 tokens 16 st .. 16 st + 15 (scores
// s[st / 2][8 (st % 2) + i], i = 2 k, 2 k + 1), rounded to fp16, and their sum (the row
// sum adds the same rounded values the PV product uses).
__device__ __forceinline__ void exp_pair(const f32x16 (&s)[2], int st, int k, float scale_log2, float off,
                                         f16x8 &pv, float &ps) {
    f16x2 pr;
    pr.x = (_Float16)exp2_fast(__builtin_fmaf(s[st / 2][8 * (st % 2) + 2 * k], scale_log2, off));
    pr.y = (_Float16)exp2_fast(__builtin_fmaf(s[st / 2][8 * (st % 2) + 2 * k + 1], scale_log2, off));
    pv[2 * k] = pr.x;
    pv[2 * k + 1] = pr.y;
    ps = __builtin_amdgcn_fdot2(pr, f16x2{(_Float16)1.0f, (_Float16)1.0f}, ps, false);
}

// A operand db of O^T += V^T P^T for the 16 tokens 16 st .. 16 st + 15 of the tile:
// rows = positions 32 db + r32, k-slot i of half hh = token 16 st + 4 hh + (i % 4)
// + 8 (i / 4), matching P's layout. Two transposed 8-byte reads: in each 16-lane group,
// source lane 4 jj + aa addresses token T + jj at positions base + 4 aa, and lane l
// receives tokens T..T+3 at position base + l.
template <int HD>
__device__ __forceinline__ f16x8 load_v_operand(const uint16_t *vr, int st, int db) {
    typedef Geo<HD> G;
    typedef __attribute__((ext_vector_type(4))) short s16x4;
    const uint16_t *p0 = vr + 16 * st * G::VROW + 32 * db;
    const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p0));
    const s16x4 hi4 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p0 + 8 * G::VROW));
    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo4), hi2 = __builtin_bit_cast(u32x2, hi4);
    return __builtin_bit_cast(f16x8, u32x4{lo2.x, lo2.y, hi2.x, hi2.y});
}

// Online softmax of the tile's scores and O^T += V^T P^T, in four 16-token steps; the
// probabilities of step st + 1 and its V operand reads are written between the products
// of step st.
template <int HD, bool BF16>
__device__ __forceinline__ void softmax_pv(Ctx<HD, BF16> &cx, const uint16_t *vl, f32x16 (&s)[2], int len,
                                           float scale_log2) {
    typedef Ctx<HD, BF16> C;
    typedef Geo<HD> G;
    constexpr int DB = C::DB;
    const int lane = threadIdx.x % kWave, hh = lane / 32, l16 = lane % 16;
    // The serial part (row maximum, rescale, first probabilities) runs at a raised wave
    // priority, lowered before the products: the SIMD's other wave then issues around
    // this chain rather than alongside it.
    __builtin_amdgcn_s_setprio(1);
    // token of s[rb][j] = 32 rb + 8 (j / 4) + 4 hh + j % 4; tokens past len do not exist
    if (len < TT) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int tok = 32 * rb + 8 * (j / 4) + 4 * hh + (j % 4);
                s[rb][j] = tok < len ? s[rb][j] : -__builtin_inff();
            }
    }
    float sm = max3(s[0][0], s[0][1], s[1][0]);
#pragma unroll
    for (int j = 2; j < 16; ++j) sm = max3(sm, s[0][j], s[1][j - 1]);
    sm = fmaxf(sm, s[1][15]);
    // the tile's row maximum of the corrected logits, log2 domain (scale > 0)
    float mt = __builtin_fmaf(sm, scale_log2, -cx.beta);
    mt = fmaxf(mt, other_half(mt));
    if (__any(mt > cx.m + kRescale)) {
        const float mnew = fmaxf(cx.m, mt);
        const float alpha = exp2_fast(cx.m - mnew);
        cx.m = mnew;
        cx.l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) cx.o[db] *= alpha;
    }
    // p = 2^(scale s - beta - m) <= 2^8
    const float off = -(cx.beta + cx.m);
    const uint16_t *vr = vl + (4 * hh + l16 / 4) * G::VROW + 16 * ((lane / 16) & 1) + 4 * (l16 % 4);
    float ps = 0.f;
    f16x8 va[2][DB], pv[2];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < DB; ++db) va[0][db] = load_v_operand<HD>(vr, 0, db);
#pragma unroll
    for (int k = 0; k < 4; ++k) exp_pair(s, 0, k, scale_log2, off, pv[0], ps);
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const int c = st & 1, n = c ^ 1;
        if (st < 3) {
#pragma unroll
            for (int db = 0; db < DB; ++db) va[n][db] = load_v_operand<HD>(vr, st + 1, db);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            cx.o[db] = mfma32_f16(va[c][db], pv[c], cx.o[db]);
            if (st < 3) {
                // 4 pairs of the next step spread over the DB products
#pragma unroll
                for (int k = db * 4 / DB; k < (db + 1) * 4 / DB; ++k) exp_pair(s, st + 1, k, scale_log2, off, pv[n], ps);
            }
        }
    }
    // keep the written order
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * DB, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, 24, 0);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        if (st < 3) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * DB, 0);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            // 4 vector instructions per product (HD 128): 6 or 8 measured slower on the long rollout
            if (st < 3) __builtin_amdgcn_sched_group_barrier(kSchedValu, 16 / DB, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    cx.l += ps;
}

// The workgroups past the attention's: the quantize-append of the current chunk, units
// (K-group fastest, then KV head, then batch) [u0, u0 + app_per_wg), one after another.
template <int HD, bool BF16>
__device__ __forceinline__ void append_units(const QuantAppendParams app, int bits, int n_groups, int n_heads,
                                             int batch, int first_wg, int per_wg) {
    typedef typename std::conditional<BF16, __bf16, _Float16>::type T;
    const int64_t U = (int64_t)n_groups * n_heads * batch;
    const int64_t u0 = (int64_t)(blockIdx.x - first_wg) * per_wg;
    const int64_t u1 = min(u0 + (int64_t)per_wg, U);
    for (int64_t u = u0; u < u1; ++u) {
        const int g = (int)(u % n_groups);
        const int64_t r = u / n_groups;
        const int h = (int)(r % n_heads), b = (int)(r / n_heads);
        if (bits == 2) qz::quant_group<T, HD, 2, kThreads, false>(app, g, h, b, n_groups);
        else qz::quant_group<T, HD, 4, kThreads, false>(app, g, h, b, n_groups);
        __syncthreads();   // the next unit reuses the group statistics in LDS
    }
}

// B operand of the per-token K columns for the lane's query: per-token K groups take
// k q2_g (k = -tau/24, q2_g the sum of the query's squares over group g's channels, or
// |q|^2 times the group's share of the channels in the isotropic form) as bf16 high and
// low parts; the compensation takes U_h^T q, the same way. Lanes of half hh hold k-slots
// 8 hh .. 8 hh + 7.
template <int HD, bool BF16>
__device__ __forceinline__ void aug_operand(Ctx<HD, BF16> &cx, const AttnParams &p, int h) {
    typedef Ctx<HD, BF16> C;
    const int hh = (threadIdx.x % kWave) / 32;
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (p.aug == AUG_TOKEN) {
        float q2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const u32x4 qw = __builtin_bit_cast(u32x4, cx.q[ks]);
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float qv = C::E::val((qw[i / 2] >> (16 * (i % 2))) & 0xffffu);
                part = __builtin_fmaf(qv, qv, part);
            }
            const int g = (16 * ks) / p.aug_kgc;
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) q2[gg] += gg == g ? part : 0.f;
        }
        float tot = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            q2[g] += other_half(q2[g]);
            tot += q2[g];
        }
        const int ng = HD / p.aug_kgc;
        const float kap = p.jensen == 0 ? 0.f : -p.beta_log2 / p.scale_log2;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float v = g < ng ? kap * (p.jensen == JENSEN_ISO ? tot / ng : q2[g]) : 0.f;
            const float vh = (float)(__bf16)v;
            const float vl = v - vh;
            x[g] = hh == 0 ? vh : vl;
            x[4 + g] = hh == 0 ? vh : 0.f;
        }
    } else if (p.aug == AUG_COMP) {
        const float *U = p.aug_basis + (size_t)h * HD * p.aug_rank;
        for (int j = 0; j < p.aug_rank; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const u32x4 qw = __builtin_bit_cast(u32x4, cx.q[ks]);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int ch = 16 * ks + 4 * (i % 4) + 2 * hh + i / 4;
                    const float qv = C::E::val((qw[i / 2] >> (16 * (i % 2))) & 0xffffu);
                    acc = __builtin_fmaf(U[(size_t)ch * p.aug_rank + j], qv, acc);
                }
            }
            acc += other_half(acc);
            const float vh = (float)(__bf16)acc;
            const float vl = acc - vh;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) x[jj] = jj == j ? (hh == 0 ? vh : vl) : x[jj];
        }
    }
    bf16x8 qa;
#pragma unroll
    for (int i = 0; i < 8; ++i) qa[i] = (__bf16)x[i];
    cx.qa = qa;
}

__device__ __forceinline__ int aug_mode(const Tile &t) {
    return t.kind() == TILE_PTOK ? AUG_TOKEN : (t.kind() == TILE_PACKED && t.comp() ? AUG_COMP : AUG_ZERO);
}

// EXACT: the all-orders Jensen form (its direct per-channel evaluation in its own instance,
// so the other forms keep their register allocation). AUG: segments with per-token K
// columns (per-token K groups, or the low-rank compensation), in an instance of their own.
template <int HD, bool BF16, bool EXACT, bool AUG>
__global__ __launch_bounds__(kThreads, 1) void attention_kernel(AttnParams p) {
    if (blockIdx.x >= (unsigned)p.n_attn_wg) {
        // a copy of the append's fields: the kernel argument itself is never addressed
        append_units<HD, BF16>(p.app, p.app_bits, p.app_groups, p.n_kv_heads, p.batch, p.n_attn_wg, p.app_per_wg);
        return;
    }
    typedef Ctx<HD, BF16> C;
    typedef typename C::vec vec;
    typedef Geo<HD> G;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * G::BUF];
    __shared__ __attribute__((aligned(16))) uint16_t augs[AUG ? 2 * TT * AROW : 8];
    __shared__ float btab_all[kWaves][32 * 32];
    // EXACT: per wave, (tau / 2) max |q| per position and its reciprocal (exact_qmax)
    __shared__ float qmt_all[EXACT ? kWaves * 2 * HD : 1];
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: wave_ok branches on scalars
    const int r32 = lane % 32, hh = lane / 32;
    const int gqa = p.n_q_heads / p.n_kv_heads;
    const int rows = gqa * p.n_q;
    __shared__ TileList tlist;

    // The workgroup's share of the work space: row block rb owns positions
    // [rb tok_pad, (rb + 1) tok_pad), position t of it standing for token t. A share is
    // cut into pieces at row-block ends; a piece that is a whole row block writes the
    // output, any other one of the two partial slots of its workgroup (0: the share's
    // first piece, 1: its last).
    // Consecutive shares (the row blocks of a head, in order) go to one XCD: workgroups are
    // dispatched to the 8 XCDs in turn (workgroup i on XCD i % 8), so workgroup i takes
    // share (i % 8) q + i / 8 (q = shares / 8; the last shares map to themselves). The row
    // blocks of a head read the same K/V stream at about the same time and then share that
    // XCD's L2 (HBM bytes per launch: long rollout 5.8x -> 1.66x the algorithmic bytes,
    // video chunk 11.2x -> 7.0x; the same time). Partial slots and the piece merge count
    // in shares.
    int share = blockIdx.x;
    {
        const int q8 = p.n_attn_wg / 8;
        if (share < 8 * q8) share = (share % 8) * q8 + share / 8;
    }
    const int64_t u0 = (int64_t)share * p.quota;
    const int64_t u1 = min(u0 + p.quota, p.work);
    for (int64_t u = u0; u < u1;) {
        const int64_t rb = u / p.tok_pad;
        const int64_t rbeg = rb * p.tok_pad;
        const int64_t ue = min(u1, rbeg + p.tok_pad);
        const int tb = (int)(u - rbeg);
        const int te = min((int)(ue - rbeg), p.n_total);
        const bool whole = tb == 0 && ue == rbeg + p.tok_pad;
        const int pslot = u == u0 ? 0 : 1;
        u = ue;
        const int bhi = (int)(rb / p.n_rb), rbi = (int)(rb - (int64_t)bhi * p.n_rb);
        const int b = bhi / p.n_kv_heads, h = bhi % p.n_kv_heads;
        const int row = rbi * BM + wave * 32 + r32;
        const bool row_ok = row < rows;
        const bool wave_ok = rbi * BM + wave * 32 < rows;
        const int hq = h * gqa + (row_ok ? row / p.n_q : 0);
        const int qi = row_ok ? row % p.n_q : 0;
        const size_t qrow = ((size_t)b * p.n_q_heads + hq) * p.n_q + qi;
        const size_t bh = (size_t)b * p.n_kv_heads + h;

        C cx;
        {
            // positions 16 ks + 8 hh + i hold channels 16 ks + 4 (i % 4) + 2 hh + i / 4:
            // element pairs (ch 2hh, 4+2hh), (8+2hh, 12+2hh), (2hh+1, 5+2hh), (9+2hh, 13+2hh)
            // dword m of a block holds channels 2m, 2m+1: this lane uses dwords hh + 2k, k = 0..3
            const uint32_t *qp = reinterpret_cast<const uint32_t *>(p.q) + qrow * (HD / 2) + hh;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                uint32_t d0 = 0u, d2 = 0u, d4 = 0u, d6 = 0u;
                if (row_ok) {
                    d0 = qp[8 * ks];
                    d2 = qp[8 * ks + 2];
                    d4 = qp[8 * ks + 4];
                    d6 = qp[8 * ks + 6];
                }
                u32x4 o;
                o.x = perm(d2, d0, 0x05040100u);
                o.y = perm(d6, d4, 0x05040100u);
                o.z = perm(d2, d0, 0x07060302u);
                o.w = perm(d6, d4, 0x07060302u);
                cx.q[ks] = __builtin_bit_cast(vec, o);
            }
        }
        if constexpr (AUG) aug_operand<HD, BF16>(cx, p, h);
        float *qmt_w = qmt_all + (EXACT ? wave * 2 * HD : 0);
        if constexpr (EXACT) exact_qmax<HD, BF16>(cx, p.half_scale, qmt_w);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) cx.o[db] = f32x16{};
        cx.btab = btab_all[wave];
        cx.m = -__builtin_inff();
        cx.l = 0.f;
        cx.beta = 0.f;

        // The piece's tiles, from lists built in bulk (all threads call fetch() together, in
        // order of i; a new list is built only after every wave has read the tiles it needs from
        // the old one: the ones it holds in cur, nxt and far).
        list_setup(p, tb, te, tlist);
        int u_total = 0;
        for (int si = 0; si <= p.n_segs; ++si) u_total += tlist.seg[si].units;
        u_total = __builtin_amdgcn_readfirstlane(u_total);
        int u_next = 0, list_base = 0, list_n = 0;
        auto fetch = [&](int i) -> Tile {
            while (i >= list_base + list_n && u_next < u_total) {
                list_base += list_n;
                u_next = __builtin_amdgcn_readfirstlane(u_next + list_build(p, tlist, u_next, u_total));
                list_n = __builtin_amdgcn_readfirstlane(tlist.n_tiles);
            }
            return i < list_base + list_n ? uniform(tlist.t[i - list_base]) : Tile::make(TILE_END, 0, 0, 0, 0, 0, 0, 16);
        };
        Tile cur = fetch(0);
        Tile nxt = fetch(1);
        Tile far = fetch(2);
        // Pipeline per tile i (one barrier per tile): tile i is computed out of LDS buffer i%2
        // while tile i+1, loaded into registers during tile i-1, is dequantized into buffer
        // (i+1)%2; then tile i+2 is loaded into the registers.
        PrefetchT<AUG> pf;
        if (cur.kind() != TILE_END) {
            prefetch_tile<HD, AUG>(pf, p, cur, bh);
            stage_tile<HD, BF16, AUG>(smem, augs, pf, stage_kind(cur), aug_mode(cur));
        }
        if (nxt.kind() != TILE_END) prefetch_tile<HD, AUG>(pf, p, nxt, bh);
        __syncthreads();
        int buf = 0, it = 0;  // cur is tile it of the piece
        while (cur.kind() != TILE_END) {
            const int sk = stage_kind(nxt);
            const uint16_t *cbuf = smem + buf * G::BUF;
            uint16_t *nbuf = smem + (buf ^ 1) * G::BUF;
            const uint16_t *acur = augs + (AUG ? buf * TT * AROW : 0);
            uint16_t *anext = augs + (AUG ? (buf ^ 1) * TT * AROW : 0);
            const int amode = aug_mode(nxt);
            if (wave_ok) {
                if (cur.kind() == TILE_PACKED) {
                    if (cur.batch()) {
                        if constexpr (EXACT) {
                            uint32_t bigm[2];
                            beta_block_poly<HD, BF16>(cx, p.segs[cur.seg()], bh, cur.g, qmt_w, bigm);
                            exact_fallback<HD, BF16>(cx, p.segs[cur.seg()], bh, cur.g, qmt_w, bigm, p.half_scale);
                        } else
                            beta_block<HD, BF16>(cx, p.segs[cur.seg()], bh, cur.g, p.jensen == JENSEN_ISO);
                    }
                    if (cur.new_group()) cx.beta = p.beta_log2 * beta_of<HD, BF16>(cx, cur.jrow());
                } else {
                    cx.beta = 0.f;
                }
                f32x16 s[2];
                if (sk == STAGE_INT2) qk_stage<HD, BF16, STAGE_INT2, AUG>(cx, cbuf, nbuf, acur, anext, pf, s, amode);
                else if (sk == STAGE_INT4) qk_stage<HD, BF16, STAGE_INT4, AUG>(cx, cbuf, nbuf, acur, anext, pf, s, amode);
                else if (sk == STAGE_RAW) qk_stage<HD, BF16, STAGE_RAW, AUG>(cx, cbuf, nbuf, acur, anext, pf, s, amode);
                else if (AUG && sk == STAGE_INT2T)
                    qk_stage<HD, BF16, STAGE_INT2T, AUG>(cx, cbuf, nbuf, acur, anext, pf, s, amode);
                else if (AUG && sk == STAGE_INT4T)
                    qk_stage<HD, BF16, STAGE_INT4T, AUG>(cx, cbuf, nbuf, acur, anext, pf, s, amode);
                else qk_stage<HD, BF16, STAGE_NONE, AUG>(cx, cbuf, nbuf, acur, anext, pf, s, amode);
                softmax_pv<HD, BF16>(cx, cbuf + G::KBUF, s, cur.len, p.scale_log2);
                if (far.kind() != TILE_END) prefetch_tile<HD, AUG>(pf, p, far, bh);
            } else {
                stage_tile<HD, BF16, AUG>(nbuf, anext, pf, sk, amode);
                if (far.kind() != TILE_END) prefetch_tile<HD, AUG>(pf, p, far, bh);
            }
            if (nxt.kind() == TILE_END) break;
            __syncthreads();
            buf ^= 1;
            cur = nxt;
            nxt = far;
            far = fetch(++it + 2);
        }

        // epilogue: lane (query r32, half hh) holds O^T[position 32 db + 8 (j/4) + 4 hh + j%4].
        // Each 32-channel block goes through the wave's Jensen table in LDS (free after the
        // tile loop; the next piece's first packed tile rebuilds it), 32 rows x 32 channels
        // with the 4-channel groups of row r at group g ^ (r % 8) (fewer bank conflicts on
        // the column writes), and leaves as 16-byte row segments. The wave alone writes and
        // reads its table; its LDS operations complete in order.
        const float lt = cx.l + other_half(cx.l);
        // a partial row leaves as block floating point: 16-bit mantissas of O 2^(15 - E),
        // 2^E the power of two above the row's largest |O| (E = 0 for a zero row)
        int pexp = 0;
        if (!whole) {
            float amax = 0.f;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(cx.o[db][j]));
            amax = fmaxf(amax, other_half(amax));
            if (amax > 0.f) pexp = ilogbf(amax) + 1;
        }
        const float scale = whole ? 1.0f / lt : ldexpf(1.0f, 15 - pexp);
        float *lo = cx.btab;
        // this lane's four chunks of a block: rows lane / 8 + 8 i, channels 4 (lane % 8) + 0..3
        const int crow = lane / 8, c4 = 4 * (lane % 8);
        const int c4s = c4 ^ (4 * (crow % 8));   // its position in the swizzled rows
        size_t dst[4];
        bool dst_ok[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rg = rbi * BM + wave * 32 + crow + 8 * i;
            dst_ok[i] = rg < rows;
            const int rgc = dst_ok[i] ? rg : 0;
            dst[i] = whole ? ((size_t)b * p.n_q_heads + h * gqa + rgc / p.n_q) * p.n_q + rgc % p.n_q
                           : ((size_t)share * 2 + pslot) * BM + (rgc - rbi * BM);
        }
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                lo[r32 * 32 + (swap_pos(8 * (j / 4) + 4 * hh + (j % 4)) ^ (4 * (r32 % 8)))] = cx.o[db][j] * scale;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(lo + (crow + 8 * i) * 32 + c4s);
                if (!dst_ok[i]) continue;
                const int ch = 32 * db + c4;
                if (!whole) {
                    uint32_t e[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        e[t] = (uint32_t)(int32_t)fminf(fmaxf(rintf(v[t]), -32767.f), 32767.f) & 0xffffu;
                    *reinterpret_cast<u32x2 *>(reinterpret_cast<uint8_t *>(p.partial) + dst[i] * PieceRow<HD>::bytes +
                                               2 * ch) = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
                } else if (p.out_dtype == DT_F32) {
                    *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.out) + dst[i] * HD + ch) = v;
                } else {
                    uint16_t e[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) e[t] = p.out_dtype == DT_BF16 ? f32_to_bf16_bits(v[t]) : f32_to_f16_bits(v[t]);
                    *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(p.out) + dst[i] * HD + ch) =
                        u32x2{(uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16)};
                }
            }
        }
        if (row_ok && hh == 0) {
            if (whole) {
                if (p.lse != nullptr) p.lse[qrow] = (cx.m + __log2f(lt)) * kLn2;
            } else {
                uint8_t *pp = reinterpret_cast<uint8_t *>(p.partial) +
                              (((size_t)share * 2 + pslot) * BM + (row - rbi * BM)) * PieceRow<HD>::bytes;
                *reinterpret_cast<f32x4 *>(pp + 2 * HD) = f32x4{cx.m, lt, __int_as_float(pexp), 0.f};
            }
        }
        // the next piece restages the LDS buffers and rebuilds the tile list
        if (u < u1) __syncthreads();
    }
}

// Merge the pieces of the row blocks that the shares split. Job y (one per workgroup of
// the attention launch) takes the row block holding position y quota if share y is the
// first to start in it; the row block's pieces are in shares w0..w1. One pass over the
// pieces with a running maximum; a thread merges 8 channels of one row (one 16-byte load
// of mantissas per piece, and the piece row's m, l and exponent). When the block's live
// rows leave threads over (few rows, e.g. decode-shaped queries cut into many pieces), NG
// groups of threads take every NG-th piece each, and their partial merges are combined
// through LDS, the same log-sum-exp way.
template <int HD>
__global__ __launch_bounds__(256) void piece_combine_kernel(AttnParams p) {
    constexpr int CPT = 8;          // channels per thread
    constexpr int TPR = HD / CPT;   // threads per row
    constexpr int RPB = 256 / TPR;  // rows per block
    constexpr int MAXG = 8;         // piece groups at most
    __shared__ float part[256][CPT + 2];   // a group's acc, then its M and L
    const int64_t U = p.quota, Np = p.tok_pad;
    const int64_t y = blockIdx.x;
    const int64_t rb = y * U / Np;
    if ((rb * Np + U - 1) / U != y) return;
    const int64_t w0 = rb * Np / U, w1 = ((rb + 1) * Np - 1) / U;
    if (w1 == w0) return;
    const int gqa = p.n_q_heads / p.n_kv_heads;
    const int rows = gqa * p.n_q;
    const int bhi = (int)(rb / p.n_rb), rbi = (int)(rb - (int64_t)bhi * p.n_rb);
    const int row_base = rbi * BM + blockIdx.y * RPB;
    const int live = min(RPB, rows - row_base);   // live rows of this block (uniform)
    if (live <= 0) return;
    const int need = live * TPR;                  // threads one pass over the pieces needs
    int NG = 1;
    while (NG < MAXG && 2 * NG * need <= 256) NG *= 2;
    const int gi = threadIdx.x / need, li = threadIdx.x % need;
    const bool active = gi < NG;
    const int r = blockIdx.y * RPB + li / TPR, c = (li % TPR) * CPT;
    const int row = rbi * BM + r;
    const int b = bhi / p.n_kv_heads, h = bhi % p.n_kv_heads;
    const size_t qrow = ((size_t)b * p.n_q_heads + h * gqa + row / p.n_q) * p.n_q + row % p.n_q;
    const uint8_t *base = reinterpret_cast<const uint8_t *>(p.partial);
    float M = -__builtin_inff(), L = 0.f;
    float acc[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) acc[i] = 0.f;
    // pieces in batches of 8 whose loads are in flight together: group gi takes pieces
    // w0 + gi, w0 + gi + NG, ...
    constexpr int NP = 8;
    if (active) {
        for (int64_t w = w0 + gi; w <= w1; w += (int64_t)NP * NG) {
            u32x4 o[NP];
            f32x4 t[NP];   // m, l, exponent bits, pad
#pragma unroll
            for (int k = 0; k < NP; ++k) {
                const int64_t ww = w + (int64_t)k * NG;
                if (ww > w1) {   // past the last piece (uniform over the group): no load
                    o[k] = u32x4{0u, 0u, 0u, 0u};
                    t[k] = f32x4{-__builtin_inff(), 0.f, 0.f, 0.f};
                    continue;
                }
                // the row block's piece in share ww is that share's first piece iff the share starts in it
                const uint8_t *pp =
                    base + (((size_t)ww * 2 + (ww * U >= rb * Np ? 0 : 1)) * BM + r) * PieceRow<HD>::bytes;
                o[k] = *reinterpret_cast<const u32x4 *>(pp + 2 * c);
                t[k] = *reinterpret_cast<const f32x4 *>(pp + 2 * HD);
            }
#pragma unroll
            for (int k = 0; k < NP; ++k) {
                const float mk = t[k][0];
                if (mk == -__builtin_inff()) continue;   // past the last piece, or a piece past the last token
                const float mn = fmaxf(M, mk);
                const float sa = exp2f(M - mn), sb = exp2f(mk - mn);
                const float so = ldexpf(sb, __float_as_int(t[k][2]) - 15);   // mantissa weight
#pragma unroll
                for (int i = 0; i < CPT; ++i) {
                    const uint32_t wd = o[k][i / 2];
                    const float mv = (float)(int16_t)(i % 2 ? wd >> 16 : wd & 0xffffu);
                    acc[i] = acc[i] * sa + mv * so;
                }
                L = L * sa + t[k][1] * sb;
                M = mn;
            }
        }
    }
    if (NG > 1) {   // uniform: the groups' partial merges meet in LDS
        if (active) {
#pragma unroll
            for (int i = 0; i < CPT; ++i) part[threadIdx.x][i] = acc[i];
            part[threadIdx.x][CPT] = M;
            part[threadIdx.x][CPT + 1] = L;
        }
        __syncthreads();
        if (gi != 0) return;
        float Mt = M;
        for (int g = 1; g < NG; ++g) Mt = fmaxf(Mt, part[g * need + li][CPT]);
        const float s0 = exp2f(M - Mt);   // a group without pieces has M = -inf: weight 0
        L *= s0;
#pragma unroll
        for (int i = 0; i < CPT; ++i) acc[i] *= s0;
        for (int g = 1; g < NG; ++g) {
            const float *pg = part[g * need + li];
            const float sg = exp2f(pg[CPT] - Mt);
            L += pg[CPT + 1] * sg;
#pragma unroll
            for (int i = 0; i < CPT; ++i) acc[i] += pg[i] * sg;
        }
        M = Mt;
    } else if (!active) {
        return;   // threads past the live rows (one group: no barrier to reach)
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int q = 0; q < CPT / 4; ++q) {
        const size_t o0 = qrow * HD + c + 4 * q;
        const f32x4 v = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]} * inv;
        if (p.out_dtype == DT_F32) {
            *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.out) + o0) = v;
        } else {
            uint16_t e[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) e[i] = p.out_dtype == DT_BF16 ? f32_to_bf16_bits(v[i]) : f32_to_f16_bits(v[i]);
            *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(p.out) + o0) =
                u32x2{(uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16)};
        }
    }
    if (c == 0 && p.lse != nullptr) p.lse[qrow] = (M + __log2f(L)) * kLn2;
}

// Merge token splits: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, in one pass with a
// running maximum over splits taken eight at a time (their loads in flight together).
template <int HD>
__global__ __launch_bounds__(HD) void combine_kernel(AttnParams p) {
    const size_t row = blockIdx.x;
    const size_t n_rows_total = (size_t)p.batch * p.n_q_heads * p.n_q;
    const int c = threadIdx.x;
    constexpr int NP = 8;
    float M = -__builtin_inff(), L = 0.f, acc = 0.f;
    for (int s0 = 0; s0 < p.n_split; s0 += NP) {
        float o[NP], m[NP], l[NP];
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            if (s0 + k >= p.n_split) {   // uniform: past the last split
                o[k] = 0.f;
                m[k] = -__builtin_inff();
                l[k] = 0.f;
                continue;
            }
            const float *pp = p.partial + dwalk::ws_row(s0 + k, n_rows_total, row) * (HD + 2);
            o[k] = pp[c];
            m[k] = pp[HD];
            l[k] = pp[HD + 1];
        }
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            if (m[k] == -__builtin_inff()) continue;   // past the last split, or a split with no tokens
            const float mn = fmaxf(M, m[k]);
            const float sa = exp2f(M - mn), sb = exp2f(m[k] - mn);
            acc = acc * sa + o[k] * sb;
            L = L * sa + l[k] * sb;
            M = mn;
        }
    }
    const float v = acc / L;
    if (p.out_dtype == DT_F32) reinterpret_cast<float *>(p.out)[row * HD + c] = v;
    else if (p.out_dtype == DT_BF16) reinterpret_cast<uint16_t *>(p.out)[row * HD + c] = f32_to_bf16_bits(v);
    else reinterpret_cast<uint16_t *>(p.out)[row * HD + c] = f32_to_f16_bits(v);
    if (c == 0 && p.lse != nullptr) p.lse[row] = (M + __log2f(L)) * kLn2;
}

template <int HD, bool BF16>
hipError_t launch_t(const AttnParams &p0, hipStream_t s) {
    AttnParams p = p0;
    const unsigned n_wg = (unsigned)((p.work + p.quota - 1) / p.quota);
    p.n_attn_wg = (int32_t)n_wg;
    unsigned n_app = 0;
    if (p.app_bits != 0) {
        // append workgroups go after the attention's: on the CUs its last round leaves idle
        // when there are a few, otherwise one per CU after it
        const int64_t U = (int64_t)p.app_groups * p.n_kv_heads * p.batch;
        const int G = device_cus();
        const int idle = (int)(n_wg % (unsigned)G) == 0 ? 0 : G - (int)(n_wg % (unsigned)G);
        const int64_t want = idle >= 4 ? idle : G;
        p.app_per_wg = (int32_t)((U + want - 1) / want);
        n_app = (unsigned)((U + p.app_per_wg - 1) / p.app_per_wg);
    }
    if (p.jensen == JENSEN_EXACT)
        hipLaunchKernelGGL((attention_kernel<HD, BF16, true, false>), dim3(n_wg + n_app), dim3(kThreads), 0, s, p);
    else if (p.aug != 0)
        hipLaunchKernelGGL((attention_kernel<HD, BF16, false, true>), dim3(n_wg + n_app), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((attention_kernel<HD, BF16, false, false>), dim3(n_wg + n_app), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.quota % p.tok_pad == 0) return e;   // no row block was split
    hipLaunchKernelGGL((piece_combine_kernel<HD>), dim3(n_wg, BM / (256 / (HD / 8))), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const AttnParams &p, hipStream_t s) {
    const unsigned n_rows_total = (unsigned)p.batch * p.n_q_heads * p.n_q;
    if (p.head_dim == 64) hipLaunchKernelGGL((combine_kernel<64>), dim3(n_rows_total), dim3(64), 0, s, p);
    else hipLaunchKernelGGL((combine_kernel<128>), dim3(n_rows_total), dim3(128), 0, s, p);
    return hipGetLastError();
}

// Compute units of the current device (one chunk-attention workgroup runs per CU); 256,
// the full gfx950 part, when there is no device to ask.
int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cached[dev] = n;
    }
    return cached[dev];
}

void attention_plan(int batch, int n_q_heads, int n_kv_heads, int head_dim, int n_q, int n_total, bool decode,
                    AttnPlan *plan) {
    *plan = AttnPlan{};
    const size_t row_bytes = (size_t)(head_dim + 2) * sizeof(float);
    if (decode) {
        int nw, wt;
        decode_plan(batch, n_kv_heads, n_total, &nw, &wt);
        plan->n_split = nw;
        plan->split_tokens = wt;
        plan->workspace_bytes = nw > 1 ? (size_t)nw * batch * n_q_heads * n_q * row_bytes : 0;
        return;
    }
    // Chunk kernel: R row blocks, each against all n_total tokens, on G CUs. When whole row
    // blocks fill the CUs' rounds to within 3 %, a workgroup takes one row block; otherwise
    // every workgroup takes an equal share of the R x n_total work (in 64-token steps, at
    // least 2 tiles), and row blocks cut between shares are merged afterwards. (A floor of 4
    // tiles left 102 of 256 CUs idle on a WindowQuant decode call, 2 row blocks x 19,648
    // positions: its attention took 40.2 against 37.2 us.)
    const long rows = (long)(n_q_heads / n_kv_heads) * n_q;
    const long n_rb = (rows + BM - 1) / BM;
    const long R = n_rb * batch * n_kv_heads;
    const long np = ((long)n_total + TT - 1) / TT * TT;
    const long G = device_cus();
    const long rounds = (R + G - 1) / G;
    const int64_t work = (int64_t)R * np;
    int64_t quota = np;
    if ((double)R / (double)(rounds * G) < 0.97) {
        quota = (work + G - 1) / G;
        quota = (quota + TT - 1) / TT * TT;
        if (quota < 2 * TT) quota = 2 * TT;
    }
    plan->n_split = 1;
    plan->n_rb = (int32_t)n_rb;
    plan->tok_pad = (int32_t)np;
    plan->quota = quota;
    plan->work = work;
    if (quota % np != 0)
        plan->workspace_bytes = (size_t)((work + quota - 1) / quota) * 2 * BM *
                                (head_dim == 64 ? PieceRow<64>::bytes : PieceRow<128>::bytes);
}

hipError_t launch_attention(const AttnParams &p, hipStream_t s) {
    if (p.decode) return launch_decode(p, s);   // (the caller launches its append after it)
    const bool bf = p.dtype == DT_BF16;
    if (p.head_dim == 64) return bf ? launch_t<64, true>(p, s) : launch_t<64, false>(p, s);
    return bf ? launch_t<128, true>(p, s) : launch_t<128, false>(p, s);
}

}  // namespace kvq
