// The decode kernel's walk over a wave's token range, and the index of every memory access
// the kernel makes, as host-and-device functions: the kernel (decode.hip) calls them, and
// a host program can run the same walk and indexing over exact-size host buffers to check
// that every access stays inside its buffer.
//
// Indexes are in units of the buffer's own element: 32-bit words for packed codes and
// {step, zero} meta, 16-bit elements for Q and the current chunk, halves of the wave's
// value tile in LDS, floats of the epilogue scratch and of the workspace.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "kvq_internal.h"

#define KVQ_HD __host__ __device__ __forceinline__

namespace kvq {
namespace dwalk {

constexpr int kDWaves = 4;
constexpr int kLanes = 64;
constexpr int TP = 64;   // tokens per step of an INT2 segment (32 for INT4)
constexpr int TR = 16;   // tokens per step of the current chunk

KVQ_HD int imin(int a, int b) { return a < b ? a : b; }
KVQ_HD int imax(int a, int b) { return a > b ? a : b; }

template <int HD> struct DGeo {
    static constexpr int NBL = HD / 64;   // 16-channel blocks per quarter row
    static constexpr int KS = HD / 32;    // k-steps of the QK product
    static constexpr int DB = HD / 16;    // 16-position blocks of O^T
    static constexpr int QV = HD / 32;    // 16-byte vectors per quarter row of 16-bit elements
    // Value row stride (halves): 8 (HD 128) or 40 (HD 64) dwords mod 64 banks, so the
    // eight 8-byte rows that half a wave reads per transposed load hit distinct banks.
    static constexpr int VROW = HD + 16;
    static constexpr int VTILE = TP * VROW;  // halves per wave
    static constexpr int OROW = HD + 4;      // epilogue scratch row (floats)
};

enum : int { ST_END = 0, ST_PACKED = 1, ST_CUR = 3 };

struct Step {
    int kind, seg, g, t, len;
    int new_group;  // first step of K-group g in this walk
    int bits;       // the segment's bit-width (16: current chunk)
};

// Walks the segments, then the current chunk, over the token range [tb, te), in steps
// that never cross a K-group. A segment's fields are read once, when the walk enters it,
// and the end of the group after next is read a group ahead, so a step inside a group
// costs a few scalar instructions. Tab::start(tab, g) reads entry g of a K-group table.
template <class Tab> struct Walker {
    int si, t, e, g, last_g, inited;
    int sbits, sng, sn;   // the current segment's bit-width, K-groups, tokens
    int ge, gen;          // end token of group g and of group g + 1
    const int32_t *tab;   // its K-group table
    KVQ_HD void init() {
        si = 0; inited = 0; last_g = -1; t = e = g = 0;
        sbits = 16; sng = sn = ge = gen = 0; tab = nullptr;
    }
    // end token of group gg, clamped: a corrupt table must not send reads outside the segment
    KVQ_HD int group_end(int gg) const {
        return gg < sng ? imin(imax(Tab::start(tab, gg + 1), 0), sn) : sn;
    }
    KVQ_HD Step next(const AttnParams &p, int tb, int te) {
        while (true) {
            if (si > p.n_segs) return Step{ST_END, 0, 0, 0, 0, 0, 16};
            if (!inited) {
                int a;
                if (si == p.n_segs) {
                    const int cb = p.n_total - p.n_cur;
                    a = imax(tb, cb) - cb;
                    e = imin(te, p.n_total) - cb;
                    sbits = 16;
                } else {
                    const SegmentView &sg = p.segs[si];
                    a = imax(tb, sg.token_begin) - sg.token_begin;
                    e = imin(te, sg.token_begin + sg.n_tokens) - sg.token_begin;
                    sbits = sg.bits;
                    sng = sg.n_kgroups;
                    sn = sg.n_tokens;
                    tab = sg.kgroup_start;
                }
                if (a >= e) { ++si; continue; }
                t = a;
                inited = 1;
                if (si < p.n_segs && sbits != 16) {
                    int lo = 0, hi = sng - 1;
                    while (lo < hi) {
                        const int mid = (lo + hi) >> 1;
                        if (Tab::start(tab, mid + 1) <= a) lo = mid + 1; else hi = mid;
                    }
                    g = lo;
                    last_g = -1;
                    ge = group_end(g);
                    gen = group_end(g + 1);
                }
            }
            if (t >= e) { ++si; inited = 0; continue; }
            if (si == p.n_segs) {
                const int len = imin(TR, e - t);
                const Step r{ST_CUR, si, 0, t, len, 0, 16};
                t += len;
                return r;
            }
            if (sbits == 16) { t = e; continue; }   // raw segments take the chunk kernel
            if (g >= sng) { t = e; continue; }
            if (ge <= t) {
                ++g;
                ge = gen;
                gen = group_end(g + 1);
                continue;
            }
            const int len = imin(sbits == 4 ? TP / 2 : TP, imin(ge, e) - t);
            const Step r{ST_PACKED, si, g, t, len, g != last_g, sbits};
            last_g = g;
            t += len;
            if (t >= ge) {
                ++g;
                ge = gen;
                gen = group_end(g + 1);
            }
            return r;
        }
    }
};

// ---- global memory. row0 = bh * capacity + step.t for packed segments.

// Q of the lane's row: 16-bit elements [q_elem, q_elem + HD / 4) (quarter j).
KVQ_HD size_t q_elem(int HD, size_t qrow, int j) { return qrow * HD + (size_t)j * (HD / 4); }

// Key codes of load b of a packed step (b < 4 INT2, b < 2 INT4): words
// [k_word, k_word + k_words(HD, bits)); rows past the step repeat its last row.
KVQ_HD int k_words(int HD, int bits) { return bits == 2 ? HD / 64 : HD / 32; }
KVQ_HD size_t k_word(int HD, int bits, size_t row0, int len, int b, int lane) {
    const int r16 = lane % 16, j = lane / 16;
    const int wpr = HD * bits / 32;
    return (row0 + imin(16 * b + r16, len - 1)) * wpr + (size_t)j * (wpr / 4);
}

// Value codes of the lane's token (INT2: token L, the whole row; INT4: token L / 2, half
// L % 2): words [v_word, v_word + v_words(HD, bits)).
KVQ_HD int v_words(int HD, int bits) { return HD / 16; }   // INT2 whole row = INT4 half row
KVQ_HD size_t v_word(int HD, int bits, size_t row0, int len, int lane) {
    if (bits == 2) return (row0 + imin(lane, len - 1)) * (HD / 16);
    return (row0 + imin(lane / 2, len - 1)) * (HD / 8) + (size_t)(lane % 2) * (HD / 16);
}
// ... and their {step, zero} words [vm_word, vm_word + vm_words(HD, bits)).
KVQ_HD int vm_words(int HD, int bits) { return bits == 2 ? HD / 32 : (HD == 128 ? 2 : 1); }
KVQ_HD size_t vm_word(int HD, int bits, size_t row0, int len, int lane) {
    if (bits == 2) return (row0 + imin(lane, len - 1)) * (HD / 32);
    return (row0 + imin(lane / 2, len - 1)) * (HD / 32) + (size_t)(lane % 2) * (HD / 64);
}

// K-group {step, zero} words of the lane's quarter: [km_word, km_word + HD / 4).
KVQ_HD size_t km_word(int HD, size_t bh, int kgroup_capacity, int g, int lane) {
    return (bh * (size_t)kgroup_capacity + g) * HD + (size_t)(lane / 16) * (HD / 4);
}

// Current chunk, row0 = bh * n_cur + step.t: keys [ck_elem, + HD / 4) (quarter j of token
// r16, token 0 of the step for lanes past it), values [cv_elem, + HD / 4) (quarter L % 4 of
// token L / 4, likewise).
KVQ_HD size_t ck_elem(int HD, size_t row0, int len, int lane) {
    const int r16 = lane % 16, j = lane / 16;
    return (row0 + (r16 < len ? r16 : 0)) * HD + (size_t)j * (HD / 4);
}
KVQ_HD size_t cv_elem(int HD, size_t row0, int len, int lane) {
    const int tr = lane / 4, qq = lane % 4;
    return (row0 + (tr < len ? tr : 0)) * HD + (size_t)qq * (HD / 4);
}

// ---- the wave's value tile in LDS (halves, [0, DGeo<HD>::VTILE)); every write is 8 halves.

// INT2: the lane's token row, 16-channel block blk (< HD / 16), halves 0..7 or 8..15.
template <int HD> KVQ_HD int vt_int2(int lane, int blk, int part) { return lane * DGeo<HD>::VROW + 16 * blk + 8 * part; }
// INT4: token L / 2, half L % 2 of the row, block hb (< HD / 32) of that half.
template <int HD> KVQ_HD int vt_int4(int lane, int hb, int part) {
    return (lane / 2) * DGeo<HD>::VROW + (lane % 2) * (HD / 2) + 16 * hb + 8 * part;
}
// current chunk: token L / 4, quarter L % 4, block bl (< NBL) of the quarter.
template <int HD> KVQ_HD int vt_cur(int lane, int bl, int part) {
    return (lane / 4) * DGeo<HD>::VROW + 16 * DGeo<HD>::NBL * (lane % 4) + 16 * bl + 8 * part;
}
// transposed read of slice h (< 2), block db (< DB): 4 halves at this index and 4 at
// index + 16 VROW.
template <int HD> KVQ_HD int vt_read(int lane, int h, int db) {
    const int l16 = lane % 16, j = lane / 16;
    const int tok0 = 32 * h + 4 * j + l16 / 4;
    return tok0 * DGeo<HD>::VROW + 16 * db + 4 * (l16 % 4);
}

// ---- epilogue: the wave's value tile read as floats ([0, VTILE / 2)): row r's O at
// channel ch, then every row's m and l.
template <int HD> KVQ_HD int epi_o(int r, int ch) { return r * DGeo<HD>::OROW + ch; }
template <int HD> KVQ_HD int epi_m(int row) { return 16 * DGeo<HD>::OROW + row; }
template <int HD> KVQ_HD int epi_l(int row) { return 16 * DGeo<HD>::OROW + 16 + row; }

// Output row of row r (< rows) of (batch b, KV head h), and the workspace row of split s:
// floats [ws_row * (HD + 2), + HD + 2) hold O, then m and l.
KVQ_HD size_t out_row(int b, int h, int r, int n_q_heads, int n_kv_heads, int n_q) {
    const int gqa = n_q_heads / n_kv_heads;
    return ((size_t)b * n_q_heads + h * gqa + r / n_q) * n_q + r % n_q;
}
KVQ_HD size_t ws_row(int split, size_t n_rows_total, size_t qrow) { return (size_t)split * n_rows_total + qrow; }

}  // namespace dwalk
}  // namespace kvq
