// layout.h -- packed-weight geometry, interval table and workspace layout of libmbk.
//
// Shared by the host-side planner/packer and the device bodies, so both read
// the same tile geometry.  Everything here is plain data and index arithmetic.
#pragma once
#include <stdint.h>

#ifndef MBK_HD
#define MBK_HD __host__ __device__ __forceinline__
#endif

namespace mbk {

constexpr int kThreads = 512;          // threads per workgroup (8 wave64)
constexpr int kWaves = kThreads / 64;
constexpr int kCW = 4;                 // compute waves (0 .. kCW-1): poll inputs, compute, publish
constexpr int kLW = kWaves - kCW;      // loader waves: stream this workgroup's future weights into LDS
constexpr int kGroups = 8;             // barrier groups: WG w belongs to group w % 8 (one per XCD
                                       // under the round-robin dispatch of an 8-XCD part)
constexpr int kMaxVec = 8192;          // largest GEMV input vector (floats) held in LDS
constexpr int kMaxGqa = 8;             // query heads per KV head handled by one attention item
constexpr int kChunk = 1024;           // bytes one wave moves with one 16-byte-per-lane load

enum Op : int32_t { OP_QKV = 0, OP_ATTN = 1, OP_O = 2, OP_GATEUP = 3, OP_DOWN = 4, OP_LMHEAD = 5 };
enum MatKind : int32_t { MAT_PLAIN = 0, MAT_QKV = 1, MAT_GATEUP = 2 };

// Weight storage formats: bf16, or OCP E4M3 8-bit codes with one
// power-of-two scale per row (fp32, in a block after each tile's codes).
enum WeightFmt : int32_t { FMT_BF16 = 0, FMT_FP8 = 1 };

// A packed matrix.  Rows (in packed order) are grouped in tiles of RT rows;
// each row's K inputs are split in groups of gv values (one 16-byte group:
// 8 bf16 or 16 fp8 codes) spread over L = 64 / RT lanes.  Chunk (tile t,
// step it, lane l) holds the group
//   packed row  t*RT + l / L,   input group  kg = (l % L) + it * L
// at byte  off + t * tb + (it * 64 + l) * 16,  IT * L >= K / gv (groups
// from K / gv on are zero padding).  So every wave-wide 16-byte load of one
// step reads 1 KiB of contiguous memory.  A tile is tb bytes: its IT KiB of
// groups, then (fp8) the fp32 scales of its RT rows at byte IT * 1024.
struct MatGeom {
    uint64_t off;    // byte offset in the packed blob
    int32_t rows;    // packed rows = ntiles * RT (rows >= logical rows)
    int32_t K;
    int32_t L, RT, IT;
    int32_t ntiles;
    int32_t kind;    // MatKind: how packed rows map to source rows
    int32_t lrt;     // log2(RT)
    int32_t fmt;     // WeightFmt
    int32_t gv;      // values per 16-byte group: 8 (bf16) or 16 (fp8)
    int32_t tb;      // bytes per tile
    int32_t pad_;
};

MBK_HD uint64_t chunk_offset(const MatGeom &g, int64_t tile, int it, int lane) {
    return g.off + (uint64_t)tile * (uint64_t)g.tb + ((uint64_t)it * 64u + (uint64_t)lane) * 16u;
}

// Byte offset of the 16-byte group kg of packed row r.
MBK_HD uint64_t row_group_offset(const MatGeom &g, int64_t r, int kg) {
    int64_t t = r / g.RT;
    int rr = (int)(r % g.RT);
    int it = kg / g.L, kl = kg % g.L;
    return chunk_offset(g, t, it, rr * g.L + kl);
}

// Byte offset of the fp32 scale of packed row r (fp8 matrices).
MBK_HD uint64_t row_scale_offset(const MatGeom &g, int64_t r) {
    return g.off + (uint64_t)(r / g.RT) * (uint64_t)g.tb + (uint64_t)g.IT * 1024u + (uint64_t)(r % g.RT) * 4u;
}

// Bytes of one tile: IT KiB of groups, plus the scale block of an fp8 tile (RT floats, 16-byte padded).
MBK_HD int tile_bytes_of(int fmt, int IT, int RT) {
    return IT * 1024 + (fmt == FMT_FP8 ? (RT * 4 + 15) / 16 * 16 : 0);
}

// Geometry rule: L is the largest power of two <= 64 dividing K/gv; operators
// whose epilogue combines two adjacent packed rows (RoPE pairs, gate/up
// pairs) need RT >= 2, so their L is capped at 32.  The planner may widen L
// for operators with few tiles (see make_geom).
MBK_HD void choose_lanes(int K, int gv, bool pairs, int *L, int *RT) {
    int kg = K / gv, l = 1;
    while (l < 64 && kg % (l * 2) == 0) l *= 2;
    if (pairs && l > 32) l = 32;
    *L = l;
    *RT = 64 / l;
}

// Source of packed row r of a fused matrix.
//  MAT_QKV: rows [0, nq*hd) are queries, then nkv*hd keys, then nkv*hd values.
//    Inside each query or key head the rows are interleaved so that packed
//    rows (2m, 2m+1) are head dims (m, m + hd/2): the pair RoPE rotates.
//  MAT_GATEUP: packed row 2i is gate row i, 2i+1 is up row i.
struct RowSrc {
    int32_t which;   // QKV: 0 q, 1 k, 2 v; GATEUP: 0 gate, 1 up; PLAIN: 0
    int32_t row;     // row inside that source matrix
};

MBK_HD RowSrc packed_row_source(int kind, int r, int hd, int nq_rows, int nkv_rows) {
    RowSrc s{0, r};
    if (kind == MAT_QKV) {
        int which = 0, base = r;
        if (r >= nq_rows + nkv_rows) { which = 2; base = r - nq_rows - nkv_rows; }
        else if (r >= nq_rows) { which = 1; base = r - nq_rows; }
        if (which < 2) {
            int h = base / hd, i = base % hd;
            base = h * hd + ((i & 1) ? (i >> 1) + hd / 2 : (i >> 1));
        }
        s.which = which;
        s.row = base;
    } else if (kind == MAT_GATEUP) {
        s.which = r & 1;
        s.row = r >> 1;
    }
    return s;
}

// One barrier interval of the static schedule (a row of the phase table).
// Its items (GEMV tiles, attention items) run on the nwg workgroups
// (wg0 + k) % n_wg, k < nwg.  GEMV: participant k owns the contiguous tile
// block [k * ntiles / nwg, (k + 1) * ntiles / nwg).  Attention: participant k
// owns items k, k + nwg, ...
struct Interval {
    int32_t op;        // Op
    int32_t layer;
    int32_t n_items;   // GEMV: tiles; attention: n_kv_heads * max_splits
    int32_t x_src;     // interval that wrote the residual-stream version read here (-1: embedding row)
    int32_t wg0, nwg;  // participating workgroups
    MatGeom mat;       // GEMV operators
    uint64_t norm_off; // RMSNorm weight folded into this interval (bf16), or ~0
    uint64_t bias_off; // Q/K/V bias (bf16, [q|k|v] natural order), or ~0
};

// One entry of a workgroup's task list: a contiguous run of GEMV tiles, or
// one attention item, of one interval.  A workgroup's tasks are stored in
// interval order; its loader waves stream the weights of every task into an
// LDS ring in that order, and its compute waves consume them in that order.
enum TaskFlag : int32_t { TASK_FIRST = 1, TASK_LAST = 2 };
struct Task {
    int32_t iv;     // interval
    int32_t a;      // GEMV: first tile; attention: item
    int32_t n;      // GEMV: tiles; attention: the item packed by attn_task_item
    int32_t flags;  // bit 0 TASK_FIRST: first task of this workgroup in iv; bit 1 TASK_LAST: last one;
                    // GEMV: bits 8.. hold the end of the workgroup's tile block
};

// Attention item `item` of an interval with ms splits per item group: KV
// head j, split s, query heads h0 .. h0 + nh - 1 of the group (one query head
// per item when hpi is 1, else all G of the KV head), packed as
// j | s << 8 | h0 << 16 | nh << 24.
MBK_HD int32_t attn_task_item(int item, int ms, int G, int hpi) {
    const int jh = item / ms, s = item % ms;
    const int j = hpi == 1 ? jh / G : jh, h0 = hpi == 1 ? jh % G : 0, nh = hpi == 1 ? 1 : G;
    return (int32_t)((uint32_t)j | ((uint32_t)s << 8) | ((uint32_t)h0 << 16) | ((uint32_t)nh << 24));
}

// Block of tiles of participant k out of nwg over ntiles tiles.
MBK_HD int block_begin(int64_t ntiles, int k, int nwg) { return (int)(ntiles * k / nwg); }

// Participant index of workgroup w in an interval, or -1.
MBK_HD int participant(const Interval &iv, int w, int n_wg) {
    const int k = (w - iv.wg0 % n_wg + n_wg) % n_wg;
    return k < iv.nwg ? k : -1;
}

// Workspace layout (bytes).  Control words get their own 256-byte lines.
// Activations handed between intervals are vectors of tagged 8-byte entries
// {fp32 value, u32 tag}: the tag names the (step, interval) that wrote the
// value, so a reader polls for exactly the version it needs.
struct WsLayout {
    uint64_t ctrl;      // [0] error flag, [1] previous argmax token, [2] LM-head arrivals,
                        // [3] token, [4] pos, [5] the step's first tag (for launches reading them here)
    uint64_t argkey;    // u64 argmax key
    uint64_t bar_global;
    uint64_t bar_group; // kGroups lines: arrival counters
    uint64_t bar_rel;   // kGroups lines: release epochs
    uint64_t merge_cnt; // n_heads lines: attention split arrivals per merge group
    uint64_t x;         // [hidden] residual stream
    uint64_t q;         // [n_heads * hd] rotated queries
    uint64_t k, v;      // [n_kv * hd] this step's rotated keys / values (fp32)
    uint64_t o;         // [n_heads * hd] attention output
    uint64_t a;         // [intermediate] silu(gate) * up
    uint64_t part;      // attention partials [n_kv][max_splits][g][hd + 4] (fp32)
    uint64_t stress;    // grid-barrier validation: 4 result words, then one epoch slot per workgroup
    uint64_t total;
};

MBK_HD uint64_t align256(uint64_t v) { return (v + 255u) & ~(uint64_t)255u; }

}  // namespace mbk
