// bodies.h -- device bodies of the decode step (gfx950, wave64).
//
// Workgroup organisation.  A workgroup (one per CU) has kWaves waves with two
// roles that never wait for each other except through LDS counters:
//  * loader waves (kCW .. kWaves-1) walk the workgroup's task list from the
//    start of the launch and copy every task's weights (or the cached keys
//    and values an attention item reads) from HBM into an LDS ring with
//    direct-to-LDS loads, as far ahead as the ring allows.  Weights do not
//    depend on activations, so their streaming runs ahead of the chain of
//    dependent intervals instead of inside it (the MegaBake article's roadmap,
//    "Checking the 5.5x": prefetching the next GEMM's weights while a block
//    waits at a barrier).
//  * compute waves (0 .. kCW-1) wait for an interval's inputs, compute its
//    tiles from the ring and publish the results.
// Loader waves count completed chunks per wave; compute waves release ring
// space by publishing how far they have consumed.  The LDS words involved
// are read by the loader through opaque LDS reads, because the compiler
// would otherwise drain every outstanding direct-to-LDS load before each
// LDS access of the loader wave.
//
// Data exchange between workgroups.  Each XCD has its own L2 and the L2s are
// not kept coherent with each other, so activations handed between
// workgroups go through the memory side with device-scope (sc1) accesses.
// Every activation vector (residual stream, queries, this step's keys and
// values, attention output, SwiGLU activations) is a vector of 8-byte
// entries {fp32 value, u32 tag} written with one 64-bit store; the tag names
// the (step, interval) that produced the value, and a reader polls exactly
// the entries it needs until they carry the tag it expects (per-phase events
// in place of grid barriers, also from the article's roadmap).  A counting
// grid barrier after every interval is kept as a mode; both modes give
// bitwise identical results.
//
// Reuse of an activation buffer is safe through the data dependencies alone:
// a vector is overwritten only by an interval that (transitively) consumed
// every output of all readers of its previous version.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace mbk {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
// LDS views: accesses through them compile to LDS instructions even where
// they are volatile or atomic (through a generic pointer they would become
// flat accesses, which wait for every outstanding global access too).
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// Loader pacing.  A loader wave learns that a chunk has landed only by waiting for its count of
// outstanding loads, so the chunks it reports complete lag the chunks it has issued by the number it keeps
// in flight; the compute waves can use only reported chunks.  The window is a trade: more chunks in
// flight per wave stream faster, but hold back more of the ring from the compute waves (measured on
// MI355X with the SmolLM-1.7B shape: 8 in flight, reported every 4, beat 24 and 8 by 9 %; 4 or 16 in
// flight were slower).
constexpr int kBatch = 4;                          // loader: chunks per wave between progress updates
constexpr int kInflight = 8;                       // loader: chunks per wave left in flight (2 batches)
constexpr uint32_t kCacheSc1 = 16;                 // cache-policy bits: device-coherent access

// Per-launch parameters (kernel argument, passed by value).
struct Params {
    const uint8_t *blob;      // packed weights + RoPE table + interval table + task lists
    const Interval *iv;       // interval table (inside blob)
    const Task *tasks;        // task lists of all workgroups (inside blob)
    const int32_t *task_idx;  // [n_wg][n_intervals + 1]: first task of workgroup w at interval i
    uint16_t *kv;             // [NL][2][nkv][S][hd] bf16
    uint8_t *ws;              // workspace
    WsLayout wl;
    float *logits;            // [V] or null
    int32_t *argmax_out;      // device int32
    const float *rope;        // [S][hd/2][2] (cos, sin)
    uint64_t *trace;          // phase timer [n_intervals][n_wg][4] or null
    MatGeom embed;            // packed tied embedding / LM head
    int32_t n_wg, n_intervals;
    int32_t H, nq, nkv, hd, I, V, S, NL;
    int32_t max_splits, gqa, attn_min_chunk, piece_pos, hd_shift;
    int32_t merge_in_o;       // 1: split partials are merged by the output projection's workgroups
    int32_t merge_dist;       // else 1: every split merges a slice of its group's outputs; 0: the last split
                              // to arrive merges them all (no workgroup waits for another inside a launch)
    int32_t attn_hpi;         // query heads per attention item: gqa (packed) or 1 (one item per query head)
    int32_t wfmt;             // WeightFmt of the projection matrices: GEMV inputs are hi/lo bf16 (bf16) or fp32 (fp8)
    // LDS offsets in bytes of the dynamic area
    int32_t lds_tasks, lds_rope, lds_qkv, lds_bias, lds_xs, lds_xres, lds_attn, lds_ring;
    int32_t ring_bytes, max_tasks;
    int32_t in_bytes, in_double;  // LDS input block [qkv | bias | xs | xres] size; 1: two copies used in turn
    float eps, scale;         // RMSNorm eps, 1/sqrt(head_dim)
    float inv_h;              // 1 / hidden
    int32_t token, pos;       // token < 0: previous device argmax
    uint32_t tag0;            // tag of this step's interval 0; interval i writes tag0 + i (nonzero)
    int32_t step_from_ws;     // 1: read token/pos/tag0 from the workspace (graph replay)
    int32_t barrier;          // 1: counting grid barrier between intervals
    uint32_t epoch_base;      // grid barriers completed on this workspace before the call
    int32_t spin_limit, skip_wg, skip_interval;
    int32_t first_iv, last_iv;
};

// LDS control words shared by the waves of a workgroup.
struct Ctl {
    alignas(16) uint32_t prog[kLW];   // loader wave w: number of its chunks known complete
    alignas(16) float ss[2][kCW];     // RMSNorm partial sums, by input-block parity
    uint32_t cons[kCW];   // compute wave c: ring consumed up to this virtual offset
    uint32_t bar;         // compute-wave barrier arrivals
    uint32_t abort;       // nonzero: leave (a bounded wait expired or the debug switch fired)
    uint64_t best[kCW];   // argmax keys
    int32_t last_s;       // attention split merge: this workgroup arrived last
};

#define MBK_DEV __device__ __forceinline__

// The launch parameters as the kernel-argument segment holds them (the
// kernels take Params as their first and only argument), through a pointer
// the compiler cannot follow from one call to the next: a loop that calls
// this once per iteration loads each field from the constant cache where it
// is used, instead of holding every field in scalar registers for the whole
// loop (which would spill them).
MBK_DEV const Params &params_opaque() {
    auto pp = (__attribute__((address_space(4))) const Params *)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(pp));
    return *(const Params *)pp;
}

// ---- access helpers ------------------------------------------------------------------------------

MBK_DEV float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
MBK_DEV float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
MBK_DEV float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (the gfx950 conversion instruction).
MBK_DEV uint16_t to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
MBK_DEV uint32_t to_bf16x2(float a, float b) {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

MBK_DEV uint32_t ldc_u(const uint32_t *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// The same for a word every lane of the wave reads at once: lane 0's value, known to the compiler as
// wave-uniform (an atomic load is otherwise taken to differ between lanes, and every branch and loop
// that depends on it becomes an exec-mask construct).
MBK_DEV uint32_t ldc_uni(const uint32_t *p) { return __builtin_amdgcn_readfirstlane(ldc_u(p)); }
MBK_DEV void stc_u(uint32_t *p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MBK_DEV uint32_t atom_add(uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

MBK_DEV auto rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}
// 16-byte device-coherent load / store (sc1) at byte offset off from base.
MBK_DEV u32x4 ldc16(const void *base, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), off, 0, 16); }
MBK_DEV void stc16(void *base, uint32_t off, u32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(base), off, 0, 16); }
MBK_DEV void stc_b16(void *base, uint32_t off, uint16_t v) {
    __builtin_amdgcn_raw_buffer_store_b16((short)v, rsrc(base), off, 0, 16);
}

template <class T> MBK_DEV T *ws_ptr(const Params &p, uint64_t off) { return (T *)(p.ws + off); }

MBK_DEV uint32_t ord_key(float f) {
    uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// LDS byte address of a pointer into LDS.
MBK_DEV uint32_t lds_addr(const void *p) { return (uint32_t)(size_t)(const lds_void_t *)p; }

// Index of the calling wave in its workgroup, known to the compiler as wave-uniform.
MBK_DEV int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// LDS accesses the compiler cannot see: used by loader waves, whose
// outstanding direct-to-LDS loads would otherwise be drained before each one.
MBK_DEV uint32_t lds_ld_opaque(const void *p) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
    return __builtin_amdgcn_readfirstlane(v);
}
MBK_DEV u32x4 lds_ld16_opaque(const void *p) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
    return v;
}
MBK_DEV void lds_st_opaque(void *p, uint32_t v) {
    asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(lds_addr(p)), "v"(v) : "memory");
}

// Control words read by every lane of a wave: the value goes to a scalar
// register, so the branches and loops that test it stay wave-uniform.

MBK_DEV uint32_t lds_ld(const uint32_t *p) { return __builtin_amdgcn_readfirstlane(*(volatile lds_u32 *)(lds_u32 *)p); }
MBK_DEV u32x4 lds_ld16(const void *p) { return *(volatile lds_u32x4 *)(lds_u32x4 *)p; }
// LDS accesses of one wave complete in order, so a control word stored after
// the data it announces is seen after that data.
MBK_DEV void lds_st(uint32_t *p, uint32_t v) { *(volatile lds_u32 *)(lds_u32 *)p = v; }

// ---- error handling ------------------------------------------------------------------------------

// Error word: set when a bounded wait expires; every wait of every workgroup gives up soon after.
MBK_DEV void set_error(const Params &p) { stc_u(ws_ptr<uint32_t>(p, p.wl.ctrl), 1u); }
MBK_DEV bool aborted(const Params &p, int it) {
    return (it & 255) == 255 && ldc_uni(ws_ptr<uint32_t>(p, p.wl.ctrl)) != 0u;
}

// ---- phase timer -----------------------------------------------------------------------------------
// Compute wave 0 stores the device wall clock (100 MHz) to the trace buffer:
// [interval][workgroup][4].  Off unless a trace buffer is bound (then the
// prologue clears this workgroup's entries first); it takes no LDS.

MBK_DEV void stamp(const Params &p, uint8_t *lds, int ivi, int k) {
    (void)lds;
    if (p.trace && threadIdx.x == 0) p.trace[((size_t)ivi * p.n_wg + blockIdx.x) * 4 + k] = wall_clock64();
}

// ---- tagged activations --------------------------------------------------------------------------

MBK_DEV uint32_t step_tag0(const Params &p) {
    return p.step_from_ws ? ldc_uni(ws_ptr<uint32_t>(p, p.wl.ctrl) + 5) : p.tag0;
}

// Tag of what interval ivi writes during the step whose interval 0 writes
// tag0.  The host hands out tags so that they are nonzero (a zeroed
// workspace never matches) and never repeat on one workspace before it is
// cleared again.
MBK_DEV uint32_t tag_of(uint32_t tag0, int ivi) { return tag0 + (uint32_t)ivi; }

// Polling loops read memory that other workgroups write: the buffer loads
// they use are not atomic, so without this compiler barrier between two
// rounds the compiler may assume a repeated read returns the same value and
// fold the loop away.  Emits no instruction.
MBK_DEV void reread() { asm volatile("" ::: "memory"); }

MBK_DEV void put(const Params &p, uint64_t base, int i, float v, uint32_t tag) {
    __hip_atomic_store(ws_ptr<uint64_t>(p, base) + i, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// 64 bytes of a tagged vector: 8 entries, tags in the odd words.
struct Group8 { u32x4 c[4]; };
MBK_DEV Group8 load8(const Params &p, uint32_t off) {
    Group8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.c[i] = ldc16(p.ws, off + 16u * i);
    return r;
}
MBK_DEV bool tagged8(const Group8 &r, uint32_t tag) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) ok = ok && r.c[i].y == tag && r.c[i].w == tag;
    return ok;
}
MBK_DEV void values8(const Group8 &r, float *v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(r.c[i].x);
        v[2 * i + 1] = __uint_as_float(r.c[i].z);
    }
}

// v[0..8) <- entries 8g..8g+7 of the tagged vector at base, once all of them
// carry `tag`.  Bounded: false when the wait expires or another wait did.
MBK_DEV bool poll8(const Params &p, uint64_t base, int g, uint32_t tag, float *v) {
    const uint32_t off = (uint32_t)(base + 64u * (uint32_t)g);
    for (int it = 0;; ++it) {
        const Group8 a = load8(p, off);
        if (tagged8(a, tag) || it >= p.spin_limit || aborted(p, it)) {
            values8(a, v);
            if (it >= p.spin_limit) set_error(p);
            return tagged8(a, tag);
        }
        reread();
    }
}

// Groups g[0 .. n) (n <= N) of the tagged vector at base: every load of a
// round is in flight at once, a round reloads only the groups still pending,
// and v[i] receives group g[i] once it carries `tag`.  Bounded like poll8.
template <int N>
MBK_DEV void poll8n(const Params &p, uint64_t base, const int *g, int n, uint32_t tag, float (*v)[8]) {
    uint32_t pending = (1u << n) - 1u;
    Group8 a[N];
    for (int it = 0;; ++it) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            if ((pending >> i) & 1u) a[i] = load8(p, (uint32_t)(base + 64u * (uint32_t)g[i]));
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (((pending >> i) & 1u) && tagged8(a[i], tag)) pending &= ~(1u << i);
        if (!pending || it >= p.spin_limit || aborted(p, it)) {
#pragma unroll
            for (int i = 0; i < N; ++i) values8(a[i], v[i]);
            if (pending && it >= p.spin_limit) set_error(p);
            return;
        }
        reread();
    }
}

// One entry of a tagged vector.
MBK_DEV bool poll1(const Params &p, uint64_t base, int i, uint32_t tag, float &v) {
    const uint64_t *e = ws_ptr<uint64_t>(p, base) + i;
    for (int it = 0;; ++it) {
        const uint64_t w = __hip_atomic_load(e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(w >> 32) == tag || it >= p.spin_limit || aborted(p, it)) {
            v = __uint_as_float((uint32_t)w);
            if (it >= p.spin_limit) set_error(p);
            return (uint32_t)(w >> 32) == tag;
        }
        reread();
    }
}

// Polls up to kPollMax 16-byte chunks of the workspace (byte offsets off[i],
// each holding two tagged entries; need[i] bit 0 / bit 1: entry 0 / 1 must
// carry the tag, bit 2: the tag is tag_b instead of tag_a) until all of them
// are ready.  Every round has all its loads in flight at once, so ready
// inputs cost one memory round trip.
constexpr int kPollMax = 12;
MBK_DEV bool poll_round(const Params &p, const uint32_t *off, const uint32_t *need, int n, uint32_t tag_a,
                        uint32_t tag_b, u32x4 *v) {
    uint32_t pending = n >= 32 ? ~0u : ((1u << n) - 1u);
    for (int it = 0;; ++it) {
#pragma unroll
        for (int i = 0; i < kPollMax; ++i)
            if ((pending >> i) & 1u) v[i] = ldc16(p.ws, off[i]);
#pragma unroll
        for (int i = 0; i < kPollMax; ++i) {
            if (!((pending >> i) & 1u)) continue;
            const uint32_t tag = (need[i] & 4u) ? tag_b : tag_a;
            const bool a = !(need[i] & 1u) || v[i].y == tag, c = !(need[i] & 2u) || v[i].w == tag;
            if (a && c) pending &= ~(1u << i);
        }
        if (!pending) return true;
        if (it >= p.spin_limit) { set_error(p); return false; }
        if (aborted(p, it)) return false;
        reread();
    }
}

// ---- grid barrier (barrier mode) -----------------------------------------------------------------
// Counting barrier with a monotonically growing arrival count (the article's
// counting grid barrier: one add per block, then wait until the count reaches
// (ordinal + 1) * workers), arranged in two levels so the adds are spread
// over 8 counters: workgroup w adds to the counter of group w % 8; the last
// arrival of a group adds to the global counter, waits for all groups and
// then publishes the epoch on its group's release word, which the other
// members poll.  Run by one thread; every wait is bounded.

MBK_DEV bool spin_until(const Params &p, const uint32_t *w, uint32_t target) {
    for (int it = 0; (int32_t)(ldc_u(w) - target) < 0; ++it) {
        if (it >= p.spin_limit) { set_error(p); return false; }
        if (aborted(p, it)) return false;
    }
    return true;
}

MBK_DEV bool grid_barrier_thread(const Params &p, uint32_t epoch) {
    const int grp = blockIdx.x % kGroups;
    const int ngroups = p.n_wg < kGroups ? p.n_wg : kGroups;
    const uint32_t members = (uint32_t)((p.n_wg - grp + kGroups - 1) / kGroups);
    uint32_t *rel = ws_ptr<uint32_t>(p, p.wl.bar_rel + 256u * grp);
    const uint32_t old = atom_add(ws_ptr<uint32_t>(p, p.wl.bar_group + 256u * grp), 1u);
    if (old == epoch * members - 1u) {
        atom_add(ws_ptr<uint32_t>(p, p.wl.bar_global), 1u);
        if (!spin_until(p, ws_ptr<uint32_t>(p, p.wl.bar_global), epoch * (uint32_t)ngroups)) return false;
        stc_u(rel, epoch);
        return true;
    }
    return spin_until(p, rel, epoch);
}

// Whole-workgroup form (the barrier microbenchmark): stores drained, one
// thread arrives and waits, the workgroup joins.
MBK_DEV bool grid_barrier(const Params &p, uint32_t epoch) {
    __shared__ int ok_s;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) ok_s = grid_barrier_thread(p, epoch);
    __syncthreads();
    return ok_s != 0;
}

// ---- reductions ----------------------------------------------------------------------------------
// Butterfly sums over groups of N consecutive lanes, all on the VALU.  Steps
// inside 16 lanes use DPP moves: after the xor-1 and xor-2 steps every quad is
// uniform, so a half-row mirror (lane i <-> 7-i) pairs quad 0 with quad 1,
// and after that a row mirror (i <-> 15-i) pairs the two halves of a 16-lane
// row.  The 16- and 32-lane steps use the gfx950 lane swaps: permlane16_swap
// returns, in every lane, its own value and the value 16 lanes away (rows
// 2k, 2k+1 exchanged), permlane32_swap likewise for the two wave halves.

template <int CTRL> MBK_DEV float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// v + (the value 16 lanes away), v + (the value 32 lanes away); max forms.
MBK_DEV float xsum16(float v) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
MBK_DEV float xsum32(float v) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
MBK_DEV float xmax16(float v) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
MBK_DEV float xmax32(float v) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

template <int N> MBK_DEV float group_sum(float v) {
    if constexpr (N >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (N >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (N >= 8) v += dpp<0x141>(v);   // row_half_mirror
    if constexpr (N >= 16) v += dpp<0x140>(v);  // row_mirror
    if constexpr (N >= 32) v = xsum16(v);
    if constexpr (N >= 64) v = xsum32(v);
    return v;
}

// The same for a group size n (a power of two up to 64) known only at run
// time: every step is computed and kept or dropped by a wave-uniform select,
// so the code has no branches.
MBK_DEV float group_sum_n(float v, int n) {
    float t = dpp<0xB1>(v);
    v = n >= 2 ? v + t : v;
    t = dpp<0x4E>(v);
    v = n >= 4 ? v + t : v;
    t = dpp<0x141>(v);
    v = n >= 8 ? v + t : v;
    t = dpp<0x140>(v);
    v = n >= 16 ? v + t : v;
    t = xsum16(v);
    v = n >= 32 ? t : v;
    t = xsum32(v);
    return n >= 64 ? t : v;
}

// ---- step inputs -----------------------------------------------------------------------------------

MBK_DEV int step_token(const Params &p) {
    int t = p.step_from_ws ? (int)ldc_uni(ws_ptr<uint32_t>(p, p.wl.ctrl) + 3) : p.token;
    if (t < 0) t = (int)ldc_uni(ws_ptr<uint32_t>(p, p.wl.ctrl) + 1);
    return t;
}
MBK_DEV int step_pos(const Params &p) {
    return p.step_from_ws ? (int)ldc_uni(ws_ptr<uint32_t>(p, p.wl.ctrl) + 4) : p.pos;
}

// ---- ring allocations ------------------------------------------------------------------------------
// Every task reads one or more allocations of the LDS ring: a GEMV task its
// tiles' weights (one contiguous byte range), an attention item its cached
// keys then values, in pieces of at most piece_pos positions.  The loader and
// compute waves derive the same sequence of allocations from the task list
// and the step's position.  An allocation is placed at the current virtual
// ring offset, or at the next multiple of the ring size if it would straddle
// the ring's end.  A GEMV task's weights take at most a third of the ring (a
// block longer than that goes in runs of whole rounds of the compute waves
// of at most a third of the ring), an attention piece at most a third (60 %
// where one piece holds a whole split); a loader
// waiting for space only ever waits for allocations it has already issued,
// which the compute waves consume and release.

// Attention split of this step: positions [0, pos] in nsplit splits of at
// most chunk positions (computed once per step: the divisions stay out of
// the per-item paths).
struct StepSplit { int Lc, chunk, nsplit; };

MBK_DEV StepSplit step_split(const Params &p, int pos) {
    StepSplit r;
    r.Lc = pos + 1;
    r.chunk = max((r.Lc + p.max_splits - 1) / p.max_splits, p.attn_min_chunk);
    r.nsplit = (r.Lc + r.chunk - 1) / r.chunk;
    return r;
}

struct Range { int t0, t1; };
MBK_DEV Range split_range(const StepSplit &ss, int s) {
    const int t0 = s * ss.chunk;
    return Range{t0, min(ss.Lc, t0 + ss.chunk)};
}

struct Alloc {
    const uint8_t *g0, *g1;   // global sources of the two segments (g1 may be null)
    uint32_t b0, b1;          // segment bytes (multiples of 16)
    uint32_t r1;              // ring offset of segment 1 inside the allocation
    uint32_t size;            // ring bytes taken
};

MBK_DEV const uint16_t *kv_block(const Params &p, int layer, int which, int j) {
    return p.kv + (((size_t)layer * 2 + which) * p.nkv + j) * p.S * p.hd;
}

// An attention item (packed by the planner into the task's n): KV head j,
// split s, query heads h0 .. h0 + nh - 1 of the group.
struct AttnItem { int j, s, h0, nh; };
MBK_DEV AttnItem attn_item(const Task &T) {
    return AttnItem{T.n & 0xff, (T.n >> 8) & 0xff, (T.n >> 16) & 0xff, (int)((uint32_t)T.n >> 24)};
}

// Cached positions [t0, min(t1, pos)) of an attention item, in pieces of
// piece_pos (a power of two) positions.
MBK_DEV int n_allocs(const Params &p, const Interval &iv, const Task &T, const StepSplit &ss) {
    if (iv.op != OP_ATTN) return 1;
    const int s = (T.n >> 8) & 0xff;
    if (s >= ss.nsplit) return 0;
    const Range r = split_range(ss, s);
    const int te = min(r.t1, ss.Lc - 1);
    return te > r.t0 ? (te - r.t0 + p.piece_pos - 1) >> __builtin_ctz((unsigned)p.piece_pos) : 0;
}

MBK_DEV Alloc task_alloc(const Params &p, const Interval &iv, const Task &T, const StepSplit &ss, int k) {
    Alloc A;
    if (iv.op != OP_ATTN) {
        const uint32_t tile_bytes = (uint32_t)iv.mat.tb;
        A.g0 = p.blob + iv.mat.off + (uint64_t)T.a * tile_bytes;
        A.b0 = (uint32_t)T.n * tile_bytes;
        A.g1 = nullptr;
        A.b1 = 0;
        A.r1 = A.b0;
        A.size = A.b0;
        return A;
    }
    const AttnItem it = attn_item(T);
    const Range r = split_range(ss, it.s);
    const int te = min(r.t1, ss.Lc - 1);
    const int pa = r.t0 + k * p.piece_pos, pb = min(te, pa + p.piece_pos);
    const uint32_t row = (uint32_t)p.hd * 2u;
    A.g0 = (const uint8_t *)kv_block(p, iv.layer, 0, it.j) + (size_t)pa * row;
    A.g1 = (const uint8_t *)kv_block(p, iv.layer, 1, it.j) + (size_t)pa * row;
    A.b0 = A.b1 = (uint32_t)(pb - pa) * row;
    A.r1 = (A.b0 + (kChunk - 1u)) & ~(kChunk - 1u);
    A.size = 2u * A.r1;
    return A;
}

// Chunks of a segment of `bytes` handled by loader wave w: chunk c of every
// segment goes to wave c % kLW.
MBK_DEV uint32_t wave_chunks(uint32_t bytes, uint32_t w) {
    static_assert((kChunk & (kChunk - 1)) == 0 && (kLW & (kLW - 1)) == 0, "shifts");
    const uint32_t nch = (bytes + (kChunk - 1u)) / (uint32_t)kChunk;
    return nch > w ? (nch - w + (uint32_t)kLW - 1u) / (uint32_t)kLW : 0u;
}

// Position in the allocation sequence: virtual offset v and its ring offset
// r = v mod R, kept together so that placing needs no division.
struct RingCursor { uint32_t v, r; };

// Places an allocation of `size` bytes: at the cursor, or at the start of the
// next turn of the ring if it would straddle the end.  Returns the ring
// offset of its start; the cursor moves to its end.
MBK_DEV uint32_t ring_place(RingCursor &c, uint32_t size, uint32_t R) {
    if (c.r + size > R) {
        c.v += R - c.r;
        c.r = 0;
    }
    const uint32_t at = c.r;
    c.v += size;
    c.r += size;
    return at;
}

// ---- loader waves ------------------------------------------------------------------------------------

// Interval descriptor ivi (uniform) from the table in the blob, through the constant address space: the
// kernels never write the table, so these are scalar loads through the scalar cache, which keeps the
// table out of LDS (the ring gets the space) and, in the loader waves, out of the count of outstanding
// vector loads.
MBK_DEV Interval interval_at(const Params &p, int ivi) {
    static_assert(sizeof(Interval) % 16 == 0, "interval size");
    constexpr int nw = (int)(sizeof(Interval) / 4);
    const auto *src = (__attribute__((address_space(4))) const uint32_t *)p.iv + ivi * nw;
    uint32_t w[nw];
#pragma unroll
    for (int i = 0; i < nw; ++i) w[i] = src[i];
    Interval v;
    __builtin_memcpy(&v, w, sizeof v);
    return v;
}

MBK_DEV Task task_opaque(const uint8_t *lds, const Params &p, int k) {
    u32x4 w = lds_ld16_opaque(lds + p.lds_tasks + 16 * k);
    Task t;
    t.iv = (int32_t)__builtin_amdgcn_readfirstlane(w.x);
    t.a = (int32_t)__builtin_amdgcn_readfirstlane(w.y);
    t.n = (int32_t)__builtin_amdgcn_readfirstlane(w.z);
    t.flags = (int32_t)__builtin_amdgcn_readfirstlane(w.w);
    return t;
}

// After each chunk a loader wave issues: every kBatch chunks it waits until at most kInflight of its chunks
// are in flight and publishes the count of its completed chunks.
MBK_DEV void batch_step(Ctl &ctl, int lw, uint32_t issued, uint32_t &published, int &inbatch) {
    static_assert(kInflight == 8, "the wait below names kInflight");
    if (++inbatch < kBatch) return;
    inbatch = 0;
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // kInflight
    if (issued > (uint32_t)kInflight && issued - (uint32_t)kInflight > published) {
        published = issued - (uint32_t)kInflight;
        lds_st_opaque(&ctl.prog[lw], published);
    }
}

// Loader wave lw's share of one segment: chunks lw, lw + kLW, ... of `bytes`
// (a multiple of 16) from global src to LDS dst, 16 bytes per lane per
// chunk; the last chunk may be partial (it counts like any other chunk).
template <int SC1>
MBK_DEV void dma_segment(const uint8_t *src, uint8_t *dst, uint32_t bytes, int lw, Ctl &ctl, uint32_t &issued,
                         uint32_t &published, int &inbatch) {
    const int lane = threadIdx.x & 63;
    const int full = (int)(bytes / kChunk);
    const uint8_t *g = src + lane * 16;
    for (int c = lw; c < full; c += kLW) {
        __builtin_amdgcn_global_load_lds((glb_void_t *)(g + (size_t)c * kChunk), (lds_void_t *)(dst + c * kChunk), 16, 0,
                                         SC1 ? (int)kCacheSc1 : 0);
        batch_step(ctl, lw, ++issued, published, inbatch);
    }
    const uint32_t rest = bytes - (uint32_t)full * kChunk;
    if (rest && full % kLW == lw) {
        if ((uint32_t)lane * 16u < rest)
            __builtin_amdgcn_global_load_lds((glb_void_t *)(g + (size_t)full * kChunk), (lds_void_t *)(dst + full * kChunk), 16,
                                             0, SC1 ? (int)kCacheSc1 : 0);
        batch_step(ctl, lw, ++issued, published, inbatch);
    }
}

// Loader wave lw: streams every allocation of tasks [0, nt) into the ring.
MBK_DEV void loader(const Params &p, uint8_t *lds, Ctl &ctl, int nt, int pos) {
    const int lw = wave_id() - kCW;
    const uint32_t R = (uint32_t)p.ring_bytes;
    uint8_t *ring = lds + p.lds_ring;
    RingCursor rc{0u, 0u};
    uint32_t issued = 0, published = 0, cons_seen = 0;
    int inbatch = 0, cur = -1;
    const StepSplit ss = step_split(p, pos);
    Interval iv;
    for (int k = 0; k < nt; ++k) {
        const Task T = task_opaque(lds, p, k);
        if (T.iv != cur) {
            iv = interval_at(p, T.iv);
            cur = T.iv;
        }
        const int na = n_allocs(p, iv, T, ss);
        const uint32_t sc1 = iv.op == OP_ATTN ? 1u : 0u;
        for (int ai = 0; ai < na; ++ai) {
            const Alloc A = task_alloc(p, iv, T, ss, ai);
            const uint32_t at = ring_place(rc, A.size, R), end = rc.v;
            if ((int32_t)(end - R - cons_seen) > 0) {
                // ring full: publish completed chunks oldest first until the
                // compute waves have released enough space
                for (int it = 0;; ++it) {
                    uint32_t c = lds_ld_opaque(&ctl.cons[0]);
#pragma unroll
                    for (int w = 1; w < kCW; ++w) {
                        const uint32_t cw = lds_ld_opaque(&ctl.cons[w]);
                        c = (int32_t)(cw - c) < 0 ? cw : c;
                    }
                    cons_seen = c;
                    if ((int32_t)(end - R - cons_seen) <= 0) break;
                    const uint32_t out = issued - published;
                    if (out > 16u) {
                        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
                        published = issued - 16u;
                    } else if (out > 8u) {
                        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
                        published = issued - 8u;
                    } else if (out > 0u) {
                        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                        published = issued;
                    }
                    if (out > 0u) {
                        lds_st_opaque(&ctl.prog[lw], published);
                        continue;
                    }
                    if (lds_ld_opaque(&ctl.abort)) return;
                    if (it >= p.spin_limit) {
                        set_error(p);
                        lds_st_opaque(&ctl.abort, 1u);
                        return;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                inbatch = 0;
            }
            uint8_t *base = ring + at;
            if (sc1) {
                dma_segment<1>(A.g0, base, A.b0, lw, ctl, issued, published, inbatch);
                if (A.b1) dma_segment<1>(A.g1, base + A.r1, A.b1, lw, ctl, issued, published, inbatch);
            } else {
                dma_segment<0>(A.g0, base, A.b0, lw, ctl, issued, published, inbatch);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_st_opaque(&ctl.prog[lw], issued);
}

// ---- compute waves: synchronisation ----------------------------------------------------------------

// Barrier among the compute waves (LDS counter).  gen counts this wave's
// barriers.  Like every wait of the compute waves it never leaves the code
// path early: when the workgroup has aborted (a bounded wait expired) it falls
// through, the step's results are void (the error word reports it) and every
// wave runs to the end of the step without waiting, so the kernel's loops keep
// a single exit.
MBK_DEV void cw_barrier(const Params &p, Ctl &ctl, uint32_t &gen) {
    gen += kCW;
    if ((threadIdx.x & 63) == 0) __atomic_fetch_add((lds_u32 *)&ctl.bar, 1u, __ATOMIC_RELAXED);
    // the first rounds spin without a pause; the abort word is looked at every 32 rounds
    for (int it = 0; (int32_t)(lds_ld(&ctl.bar) - gen) < 0; ++it) {
        if ((it & 31) == 31) {
            if (lds_ld(&ctl.abort)) return;
            if (it >= p.spin_limit) {
                set_error(p);
                lds_st(&ctl.abort, 1u);
                return;
            }
        }
        if (it >= 64) __builtin_amdgcn_s_sleep(1);
    }
}

// Position of the compute waves in the allocation sequence.
struct RingPos {
    RingCursor cur;
    uint32_t cum[kLW];    // chunks of each loader wave up to the current allocation
    uint32_t seen[kLW];   // loader progress last read from LDS
};

// All loader waves' progress with one LDS read.
MBK_DEV void read_prog(Ctl &ctl, uint32_t *out) {
    static_assert(kLW == 4, "one 16-byte read of the loader progress");
    const u32x4 v = lds_ld16(ctl.prog);
    out[0] = __builtin_amdgcn_readfirstlane(v.x);
    out[1] = __builtin_amdgcn_readfirstlane(v.y);
    out[2] = __builtin_amdgcn_readfirstlane(v.z);
    out[3] = __builtin_amdgcn_readfirstlane(v.w);
}

// Places the next allocation; waits until the loader waves have completed it
// (falls through once the workgroup has aborted).  Returns its ring offset.
MBK_DEV uint32_t ring_acquire(const Params &p, Ctl &ctl, RingPos &rp, const Alloc &A) {
    const uint32_t start = ring_place(rp.cur, A.size, (uint32_t)p.ring_bytes);
#pragma unroll
    for (int w = 0; w < kLW; ++w) rp.cum[w] += wave_chunks(A.b0, (uint32_t)w) + wave_chunks(A.b1, (uint32_t)w);
    // the loader is usually far ahead: the progress read last time often covers this allocation
    for (int it = 0;; ++it) {
        bool ready = true;
#pragma unroll
        for (int w = 0; w < kLW; ++w) ready = ready && (int32_t)(rp.seen[w] - rp.cum[w]) >= 0;
        if (ready) return start;
        if (it > 0) {
            if (lds_ld(&ctl.abort)) return start;
            if (it >= p.spin_limit) {
                set_error(p);
                lds_st(&ctl.abort, 1u);
                return start;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        read_prog(ctl, rp.seen);
    }
}

MBK_DEV void ring_release(Ctl &ctl, const RingPos &rp) { lds_st(&ctl.cons[wave_id()], rp.cur.v); }

// ---- GEMV input vectors ------------------------------------------------------------------------------
// GEMV input vectors live in LDS as bf16 pairs: each 8-element group g is 32
// bytes, [hi pairs | lo pairs] with hi = bf16(x), lo = bf16(x - hi), so that
// hi + lo carries ~17 significant bits and the bf16 dot-product instruction
// (fp32 accumulation) consumes weights and activations without conversions.
// RMS-normalised inputs are stored without the 1/rms factor, which is applied
// to the row sums.

MBK_DEV void split8_store(float *dst, const float *v) {
    u32x4 h, l;
    h.x = to_bf16x2(v[0], v[1]);
    h.y = to_bf16x2(v[2], v[3]);
    h.z = to_bf16x2(v[4], v[5]);
    h.w = to_bf16x2(v[6], v[7]);
    l.x = to_bf16x2(v[0] - bf_lo(h.x), v[1] - bf_hi(h.x));
    l.y = to_bf16x2(v[2] - bf_lo(h.y), v[3] - bf_hi(h.y));
    l.z = to_bf16x2(v[4] - bf_lo(h.z), v[5] - bf_hi(h.z));
    l.w = to_bf16x2(v[6] - bf_lo(h.w), v[7] - bf_hi(h.w));
    *(u32x4 *)dst = h;
    *(u32x4 *)(dst + 4) = l;
}

// GEMV input group g of 8 values: hi/lo bf16 pairs for bf16 weights, the 8 fp32 values for fp8 weights
// (whose products are formed in fp32 after the codes are widened).
MBK_DEV void stage8(const Params &p, float *dst, const float *v);

MBK_DEV void unpack8(const u32x4 &w, float *v) {
    v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
    v[4] = bf_lo(w.z); v[5] = bf_hi(w.z); v[6] = bf_lo(w.w); v[7] = bf_hi(w.w);
}

MBK_DEV void store8(float *dst, const float *v) {
    *(float4 *)dst = make_float4(v[0], v[1], v[2], v[3]);
    *(float4 *)(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

MBK_DEV void stage8(const Params &p, float *dst, const float *v) {
    if (p.wfmt == FMT_FP8) store8(dst, v);
    else split8_store(dst, v);
}

// xs <- hi/lo of (v * w) for the residual stream v (tagged, or the embedding
// row of `token`) and the bf16 norm weight w; returns this thread's part of
// sum(v^2).  Threads [tid, nt).
MBK_DEV float norm_input(const Params &p, float *xs, bool from_embed, int token, uint32_t tag, uint64_t norm_off,
                         int K, int tid, int nt) {
    float ss = 0.f;
    for (int g = tid; g < K / 8; g += nt) {
        float v[8], w[8];
        // the norm weights (and the embedding row) are requested before the poll, so they arrive with it
        const u32x4 wn = *(const u32x4 *)(p.blob + norm_off + 16u * g);
        if (from_embed) unpack8(*(const u32x4 *)(p.blob + row_group_offset(p.embed, token, g)), v);
        else poll8(p, p.wl.x, g, tag, v);
        unpack8(wn, w);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ss += v[e] * v[e];
            v[e] *= w[e];
        }
        stage8(p, xs + 8 * g, v);
    }
    return ss;
}

// xs <- hi/lo pairs of the tagged vector at base (threads [tid, nt)).  A
// thread polls all its groups (up to 4 per round: the widest inputs, 8192
// entries over 256 threads, have 4) at once, so a wide input costs one wait
// for its last group rather than one per group.
MBK_DEV void plain_input(const Params &p, float *xs, uint64_t base, uint32_t tag, int K, int tid, int nt) {
    constexpr int kG = 4;
    const int ng = K / 8;
    if (ng <= nt) {  // one group per thread at most
        if (tid < ng) {
            float v[8];
            poll8(p, base, tid, tag, v);
            stage8(p, xs + 8 * tid, v);
        }
        return;
    }
    for (int g0 = tid; g0 < ng; g0 += kG * nt) {
        int g[kG], n = 0;
#pragma unroll
        for (int i = 0; i < kG; ++i) {
            g[i] = g0 + i * nt;
            if (g[i] < ng) n = i + 1;
        }
        float v[kG][8];
        poll8n<kG>(p, base, g, n, tag, v);
#pragma unroll
        for (int i = 0; i < kG; ++i)
            if (i < n) stage8(p, xs + 8 * g[i], v[i]);
    }
}

// xs <- hi/lo pairs of the attention output, merged from the split partials
// (log-sum-exp merge in split order): thread u takes query head u / (hd/8),
// dims 8 * (u % (hd/8)) .. + 8.  Threads [tid, nt).
template <int G>
MBK_DEV void merge_input(const Params &p, float *xs, uint32_t tag, int nsplit, int tid, int nt) {
    const int hd = p.hd, gsh = p.hd_shift - 3, gpr = 1 << gsh;
    constexpr int kPer = kPollMax / 5;  // splits per polling round: {max, sum} chunk + 4 chunks of acc
    for (int u = tid; u < p.nq * gpr; u += nt) {
        const int h = u >> gsh, g = u & (gpr - 1), j = h / G, hh = h - j * G;
        float M = -INFINITY, L = 0.f, a[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = 0.f;
        for (int s0 = 0; s0 < nsplit; s0 += kPer) {
            const int ns = min(kPer, nsplit - s0);
            uint32_t off[kPollMax], need[kPollMax];
            u32x4 v[kPollMax];
#pragma unroll
            for (int i = 0; i < kPollMax; ++i) { off[i] = 0; need[i] = 0; }
            // fixed trip counts, so the arrays stay in registers
#pragma unroll
            for (int q = 0; q < kPer; ++q) {
                if (q >= ns) break;
                const uint32_t e0 = (uint32_t)(((j * p.max_splits + s0 + q) * G + hh) * (hd + 2));
                off[5 * q] = (uint32_t)p.wl.part + 8u * (e0 + (uint32_t)hd);
                need[5 * q] = 3u;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    off[5 * q + 1 + c] = (uint32_t)p.wl.part + 8u * (e0 + 8u * (uint32_t)g) + 16u * c;
                    need[5 * q + 1 + c] = 3u;
                }
            }
            poll_round(p, off, need, 5 * ns, tag, tag, v);
#pragma unroll
            for (int q = 0; q < kPer; ++q) {
                if (q >= ns) break;
                const float m2 = __uint_as_float(v[5 * q].x), l2 = __uint_as_float(v[5 * q].z);
                float w[8];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    w[2 * c] = __uint_as_float(v[5 * q + 1 + c].x);
                    w[2 * c + 1] = __uint_as_float(v[5 * q + 1 + c].z);
                }
                const float mn = fmaxf(M, m2);
                const float c1 = __expf(M - mn), c2 = __expf(m2 - mn);
                L = L * c1 + l2 * c2;
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] = a[e] * c1 + w[e] * c2;
                M = mn;
            }
        }
        const float inv = 1.f / L;
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] *= inv;
        stage8(p, xs + 8 * u, a);
    }
}

// ---- GEMV tile ---------------------------------------------------------------------------------------
// A tile is RT packed rows; lane l covers row l / L and input groups
// (l % L) + it * L, it < IT, reading the 16-byte chunk at it * 1 KiB + l * 16
// of the tile's weights in the ring.  The row sum is reduced over its L lanes;
// every lane returns the sum of its row.

MBK_DEV float dot2(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, x), acc, false);
}

// B chunks at once: all LDS reads (weights, then the hi/lo input groups) are
// issued before the first product, so their latencies overlap.
template <int B>
MBK_DEV void gemv_batch(const u32x4 *w, const float *xs, int it, int L, int kl, float *a) {
    u32x4 c[B], h[B], l[B];
#pragma unroll
    for (int u = 0; u < B; ++u) c[u] = w[(it + u) * 64];
#pragma unroll
    for (int u = 0; u < B; ++u) {
        const float *xv = xs + (kl + (it + u) * L) * 8;
        h[u] = *(const u32x4 *)xv;
        l[u] = *(const u32x4 *)(xv + 4);
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
        a[0] = dot2(c[u].x, h[u].x, a[0]);
        a[1] = dot2(c[u].y, h[u].y, a[1]);
        a[2] = dot2(c[u].z, h[u].z, a[2]);
        a[3] = dot2(c[u].w, h[u].w, a[3]);
        a[0] = dot2(c[u].x, l[u].x, a[0]);
        a[1] = dot2(c[u].y, l[u].y, a[1]);
        a[2] = dot2(c[u].z, l[u].z, a[2]);
        a[3] = dot2(c[u].w, l[u].w, a[3]);
    }
}

MBK_DEV float gemv_tile(const MatGeom &g, const uint8_t *wt, const float *xs) {
    const int lane = threadIdx.x & 63, kl = lane & (g.L - 1);
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    const u32x4 *w = (const u32x4 *)wt + lane;
    int it = 0;
    for (; it + 8 <= g.IT; it += 8) gemv_batch<8>(w, xs, it, g.L, kl, a);
    if (it + 4 <= g.IT) { gemv_batch<4>(w, xs, it, g.L, kl, a); it += 4; }
    if (it + 2 <= g.IT) { gemv_batch<2>(w, xs, it, g.L, kl, a); it += 2; }
    if (it < g.IT) gemv_batch<1>(w, xs, it, g.L, kl, a);
    return group_sum_n((a[0] + a[1]) + (a[2] + a[3]), g.L);
}

// fp8 tile: the same lanes and steps over groups of 16 E4M3 codes; each code is widened to fp32 by the
// hardware conversion (OCP E4M3 on gfx950) and multiplied with the fp32 input (the products carry the
// code's 4 significant bits times the input's 24).  The row's scale is applied by the epilogue.
template <int B>
MBK_DEV void gemv_batch_fp8(const u32x4 *w, const float *xs, int it, int L, int kl, float *a) {
    u32x4 c[B];
    float4 x[B][4];
#pragma unroll
    for (int u = 0; u < B; ++u) c[u] = w[(it + u) * 64];
#pragma unroll
    for (int u = 0; u < B; ++u) {
        const float4 *xv = (const float4 *)(xs + (kl + (it + u) * L) * 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) x[u][j] = xv[j];
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
        const uint32_t cw[4] = {c[u].x, c[u].y, c[u].z, c[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[j], false);   // codes 4j, 4j + 1
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[j], true);    // codes 4j + 2, 4j + 3
            a[j] = fmaf(lo[0], x[u][j].x, a[j]);
            a[j] = fmaf(lo[1], x[u][j].y, a[j]);
            a[j] = fmaf(hi[0], x[u][j].z, a[j]);
            a[j] = fmaf(hi[1], x[u][j].w, a[j]);
        }
    }
}

MBK_DEV float gemv_tile_fp8(const MatGeom &g, const uint8_t *wt, const float *xs) {
    const int lane = threadIdx.x & 63, kl = lane & (g.L - 1);
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    const u32x4 *w = (const u32x4 *)wt + lane;
    int it = 0;
    for (; it + 4 <= g.IT; it += 4) gemv_batch_fp8<4>(w, xs, it, g.L, kl, a);
    if (it + 2 <= g.IT) { gemv_batch_fp8<2>(w, xs, it, g.L, kl, a); it += 2; }
    if (it < g.IT) gemv_batch_fp8<1>(w, xs, it, g.L, kl, a);
    // the row's power-of-two scale, from the tile's scale block
    const float scale = ((const float *)(wt + g.IT * 1024))[lane >> (6 - g.lrt)];
    return group_sum_n((a[0] + a[1]) + (a[2] + a[3]), g.L) * scale;
}

// ---- GEMV epilogues (per tile; row sums in every lane of the row) ------------------------------------

struct StepCtx {
    int pos, token;
    StepSplit ss;    // this step's attention split
    uint32_t tag0;   // tag of this step's interval 0
    float rnorm;     // 1/rms of the interval's normalised input (1 when not normalised)
    uint32_t gen;    // compute-wave barrier generation
    uint64_t best;   // this lane's argmax key (LM head)
    int blk0;        // first tile of this workgroup's block in the current interval
    int in;          // byte offset of the input block in use
    uint32_t nin;    // input blocks loaded so far
};

// Q/K/V: bias, RoPE on query/key pairs (packed rows 2m, 2m+1 are head dims
// m, m + hd/2: lanes L apart); queries and this step's keys/values published
// as tagged vectors, keys/values appended to the cache at slot pos.
MBK_DEV void epi_qkv(const Params &p, const Interval &iv, const uint8_t *lds, int t, float y, const StepCtx &sc,
                     uint32_t tag) {
    const MatGeom &g = iv.mat;
    const int lane = threadIdx.x & 63, hd = p.hd, hs = p.hd_shift, Q = p.nq * hd, KVr = p.nkv * hd, half = hd / 2;
    const int row = t * g.RT + (lane >> (6 - g.lrt));
    const bool valid = (lane & (g.L - 1)) == 0 && row < g.rows;
    // source row of packed row `row` (the packer's interleave: packed rows 2m, 2m+1 of a query or key
    // head are its dims m and m + hd/2)
    RowSrc s;
    {
        const int r = valid ? row : 0;
        s.which = r >= Q + KVr ? 2 : (r >= Q ? 1 : 0);
        const int base = r - (s.which == 0 ? 0 : (s.which == 1 ? Q : Q + KVr));
        const int i = base & (hd - 1);
        s.row = s.which == 2 ? base : (base & ~(hd - 1)) + ((i & 1) ? (i >> 1) + half : (i >> 1));
    }
    if (iv.bias_off != ~(uint64_t)0 && valid) {
        const float *bias = (const float *)(lds + p.lds_bias + sc.in);
        y += bias[(s.which == 0 ? 0 : (s.which == 1 ? Q : Q + KVr)) + s.row];
    }
    const float partner = __shfl_xor(y, g.L);  // row ^ 1
    if (!valid) return;
    const int pos = sc.pos;
    if (s.which == 2) {
        uint16_t *vc = p.kv + ((size_t)iv.layer * 2 + 1) * p.nkv * p.S * hd;
        const int j = s.row >> hs, d = s.row & (hd - 1);
        put(p, p.wl.v, s.row, y, tag);
        stc_b16(vc, (uint32_t)((((size_t)j * p.S + pos) * hd + d) * 2u), to_bf16(y));
        return;
    }
    if (row & 1) return;  // the odd row is the partner of this pair
    const int h = s.row >> hs, m = s.row & (hd - 1);  // m < hd/2
    const float2 cs = ((const float2 *)(lds + p.lds_rope))[m];
    const float r0 = y * cs.x - partner * cs.y, r1 = partner * cs.x + y * cs.y;
    if (s.which == 0) {
        put(p, p.wl.q, h * hd + m, r0, tag);
        put(p, p.wl.q, h * hd + m + half, r1, tag);
    } else {
        uint16_t *kc = p.kv + ((size_t)iv.layer * 2 + 0) * p.nkv * p.S * hd;
        put(p, p.wl.k, h * hd + m, r0, tag);
        put(p, p.wl.k, h * hd + m + half, r1, tag);
        const size_t base = ((size_t)h * p.S + pos) * hd;
        stc_b16(kc, (uint32_t)((base + m) * 2u), to_bf16(r0));
        stc_b16(kc, (uint32_t)((base + m + half) * 2u), to_bf16(r1));
    }
}

// Runs one tile and its epilogue.
MBK_DEV void gemv_tile_op(const Params &p, const Interval &iv, const uint8_t *lds, const uint8_t *wt, int t,
                          StepCtx &sc, uint32_t tag) {
    const MatGeom &g = iv.mat;
    const float *xs = (const float *)(lds + p.lds_xs + sc.in);
    float y = (g.fmt == FMT_FP8 ? gemv_tile_fp8(g, wt, xs) : gemv_tile(g, wt, xs)) * sc.rnorm;
    const int lane = threadIdx.x & 63;
    const int row = t * g.RT + (lane >> (6 - g.lrt));
    const bool lead = (lane & (g.L - 1)) == 0 && row < g.rows;
    switch (iv.op) {
        case OP_QKV: epi_qkv(p, iv, lds, t, y, sc, tag); break;
        case OP_O:
        case OP_DOWN: {
            const float *xres = (const float *)(lds + p.lds_xres + sc.in);
            if (lead) put(p, p.wl.x, row, xres[row - sc.blk0 * g.RT] + y, tag);
            break;
        }
        case OP_GATEUP: {
            const float up = __shfl_xor(y, g.L);
            if (lead && !(row & 1)) put(p, p.wl.a, row >> 1, __fdividef(y, 1.f + __expf(-y)) * up, tag);
            break;
        }
        default: {  // LM head
            if (lead) {
                if (p.logits) p.logits[row] = y;
                const uint64_t key = ((uint64_t)ord_key(y) << 32) | (uint64_t)(0xffffffffu - (uint32_t)row);
                sc.best = key > sc.best ? key : sc.best;
            }
            break;
        }
    }
}

// Greedy argmax: the compute waves' keys meet in LDS, one 64-bit atomic max
// per workgroup; the last participant to arrive publishes the index and
// clears the key and the count for the next step.
MBK_DEV void argmax_publish(const Params &p, const Interval &iv, Ctl &ctl, StepCtx &sc) {
    uint64_t best = sc.best;
    for (int m = 1; m < 64; m <<= 1) {
        const uint64_t o = ((uint64_t)__shfl_xor((uint32_t)(best >> 32), m) << 32) | __shfl_xor((uint32_t)best, m);
        best = o > best ? o : best;
    }
    const int cw = wave_id();
    if ((threadIdx.x & 63) == 0) ctl.best[cw] = best;
    cw_barrier(p, ctl, sc.gen);
    if (threadIdx.x == 0) {
        for (int i = 0; i < kCW; ++i) best = ctl.best[i] > best ? ctl.best[i] : best;
        uint64_t *key = ws_ptr<uint64_t>(p, p.wl.argkey);
        if (best) __hip_atomic_fetch_max(key, best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        uint32_t *ctrl = ws_ptr<uint32_t>(p, p.wl.ctrl);
        if (atom_add(ctrl + 2, 1u) == (uint32_t)iv.nwg - 1u) {
            const uint64_t k = __hip_atomic_load(key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int32_t idx = (int32_t)(0xffffffffu - (uint32_t)k);
            p.argmax_out[0] = idx;
            stc_u(ctrl + 1, (uint32_t)idx);
            __hip_atomic_store(key, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            stc_u(ctrl + 2, 0u);
        }
    }
    sc.best = 0;
}

// ---- interval inputs (compute waves, threads [0, kCW * 64)) ------------------------------------------

// Returns this thread's part of the RMSNorm sum of squares (0 if none).  T is
// the workgroup's first task of the interval.
template <int G>
MBK_DEV float gemv_inputs(const Params &p, const Interval &iv, const Task &T, int ivi, uint8_t *lds, StepCtx &sc) {
    const int tid = threadIdx.x, nt = kCW * 64;
    float *xs = (float *)(lds + p.lds_xs + sc.in);
    const uint32_t xtag = iv.x_src < 0 ? 0u : tag_of(sc.tag0, iv.x_src);
    // groups past the input (padding of widened tiles) are zero
    for (int g = iv.mat.K / 8 + tid; g < iv.mat.IT * iv.mat.L * (iv.mat.gv / 8); g += nt) {
        *(u32x4 *)(xs + 8 * g) = (u32x4){0u, 0u, 0u, 0u};
        *(u32x4 *)(xs + 8 * g + 4) = (u32x4){0u, 0u, 0u, 0u};
    }
    switch (iv.op) {
        case OP_O:
        case OP_DOWN: {
            // residual rows of this workgroup's tile block
            const MatGeom &g = iv.mat;
            const int b0 = T.a, b1 = T.flags >> 8;  // this workgroup's tile block
            sc.blk0 = b0;
            float *xres = (float *)(lds + p.lds_xres + sc.in);
            const int r0 = b0 * g.RT, r1 = min(b1 * g.RT, g.rows);
            // the last threads take the rows: the input vector's groups go to the first ones, so
            // both reads are in flight together
            for (int r = r0 + (nt - 1 - tid); r < r1; r += nt) {
                if (iv.x_src < 0) {
                    const uint16_t *e = (const uint16_t *)(p.blob + row_group_offset(p.embed, sc.token, r >> 3));
                    xres[r - r0] = bf16f(e[r & 7]);
                } else {
                    poll1(p, p.wl.x, r, xtag, xres[r - r0]);
                }
            }
            if (iv.op == OP_O && p.merge_in_o) merge_input<G>(p, xs, tag_of(sc.tag0, ivi - 1), sc.ss.nsplit, tid, nt);
            else if (iv.op == OP_O) plain_input(p, xs, p.wl.o, tag_of(sc.tag0, ivi - 1), p.nq * p.hd, tid, nt);
            else plain_input(p, xs, p.wl.a, tag_of(sc.tag0, ivi - 1), p.I, tid, nt);
            return 0.f;
        }
        case OP_QKV: {
            if (iv.bias_off == ~(uint64_t)0) return norm_input(p, xs, iv.x_src < 0, sc.token, xtag, iv.norm_off, p.H, tid, nt);
            // Q/K/V bias to LDS (fp32), 8 values per 16-byte load; the first load of each thread is
            // in flight while the residual stream is polled
            const int nb8 = (p.nq + 2 * p.nkv) * p.hd / 8;
            const u32x4 *bsrc = (const u32x4 *)(p.blob + iv.bias_off);
            float *bias = (float *)(lds + p.lds_bias + sc.in);
            u32x4 first = {0u, 0u, 0u, 0u};
            if (tid < nb8) first = bsrc[tid];
            const float ss = norm_input(p, xs, iv.x_src < 0, sc.token, xtag, iv.norm_off, p.H, tid, nt);
            for (int i = tid; i < nb8; i += nt) {
                float v[8];
                unpack8(i == tid ? first : bsrc[i], v);
                store8(bias + 8 * i, v);
            }
            return ss;
        }
        default:  // gate/up and LM head: RMS-normalised residual stream
            return norm_input(p, xs, false, 0, xtag, iv.norm_off, p.H, tid, nt);
    }
}

// Attention item inputs: the G queries of its KV head, pre-scaled, and the
// key and value appended this step, rounded to bf16 exactly as the cache
// holds them.  LDS at lds_qkv: [G][hd] queries, [hd] key, [hd] value.
template <int G>
MBK_DEV void attn_inputs(const Params &p, const Task &T, int ivi, uint8_t *lds, const StepCtx &sc) {
    const int tid = threadIdx.x, nt = kCW * 64;
    const AttnItem it = attn_item(T);
    const int hd = p.hd, kg = hd >> 3, qg = it.nh * kg;
    const uint32_t tag = tag_of(sc.tag0, ivi - 1);
    float *dst = (float *)(lds + p.lds_qkv + sc.in);
    for (int g = tid; g < qg + 2 * kg; g += nt) {
        float v[8];
        if (g < qg) {
            // queries of heads h0 .. h0 + nh - 1 of group j, at [0, nh)
            poll8(p, p.wl.q, (it.j * G + it.h0) * kg + g, tag, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= p.scale;
            store8(dst + 8 * g, v);
        } else {
            const bool key = g < qg + kg;
            const int gg = g - qg - (key ? 0 : kg);
            poll8(p, key ? p.wl.k : p.wl.v, it.j * kg + gg, tag, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = bf16f(to_bf16(v[e]));
            store8(dst + G * hd + (key ? 0 : hd) + 8 * gg, v);
        }
    }
}

// ---- attention ---------------------------------------------------------------------------------------
// Decode attention for KV head j over the cached positions of one split, for
// one of its query heads (the default item) or for all G of them packed
// together so each key and value is read once (README mirror, "Current
// status": flash decoding, query heads sharing a KV head packed at long
// context; the planner chooses, see the attention items rule in mbk.hip).
// Lane (slot, dl) of a compute wave
// takes one position per block and head dims dl*8 .. dl*8+7 (LP = hd/8
// lanes per position); the compute waves take alternate blocks.  Cached
// positions arrive in the ring pieces; the position appended this step is
// read from LDS.  Every lane keeps the running maximum, sum and weighted
// values of its own positions (online softmax in one pass over the keys and
// values: a new maximum rescales what the lane holds; a lane folds several
// positions in at once, so their scores are formed side by side), so neither
// the lanes nor the waves wait for one another inside an item; at its end
// the slots of a wave, then the waves in LDS, are combined with the
// log-sum-exp rule, like the partials of different splits.

// 8 floats from LDS.
MBK_DEV void load8f(const float *src, float *f) {
    const float4 a = *(const float4 *)src, b = *(const float4 *)(src + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Sum (max) over the slots of a wave: the lanes with the same lane % LP.
// Inside a 16-lane row the slots are combined by rotating the row by 2, 4
// and 8 lanes (each step doubles the slots covered), then rows by the lane
// swaps (only the steps LP needs).
template <int LP> MBK_DEV float slot_sum(float v) {
    if constexpr (LP <= 1) v += dpp<0x121>(v);   // row_ror:1
    if constexpr (LP <= 2) v += dpp<0x122>(v);   // row_ror:2
    if constexpr (LP <= 4) v += dpp<0x124>(v);   // row_ror:4
    if constexpr (LP <= 8) v += dpp<0x128>(v);   // row_ror:8
    return xsum32(xsum16(v));
}
template <int LP> MBK_DEV float slot_max(float v) {
    if constexpr (LP <= 1) v = fmaxf(v, dpp<0x121>(v));
    if constexpr (LP <= 2) v = fmaxf(v, dpp<0x122>(v));
    if constexpr (LP <= 4) v = fmaxf(v, dpp<0x124>(v));
    if constexpr (LP <= 8) v = fmaxf(v, dpp<0x128>(v));
    return xmax32(xmax16(v));
}

// Tagged 16-byte store of entries i, i+1 (i even).
MBK_DEV void put2(const Params &p, uint64_t base, int i, float a, float b, uint32_t tag) {
    stc16(p.ws, (uint32_t)(base + 8u * (uint32_t)i), (u32x4){__float_as_uint(a), tag, __float_as_uint(b), tag});
}

// Split-context merge done by all the splits of a merge group at once (gh query heads hb .. hb + gh - 1
// of KV head j, their outputs taken in pairs of dims): split s merges pairs s, s + nsplit, ... from
// the tagged partials {acc[hd] | max, sum} of every split, in split order with the largest maximum
// first (the same arithmetic as a single merging workgroup, so the result does not depend on which
// workgroup merges), and publishes them as the attention output.  A pair's inputs are polled by one
// thread per split; scr holds [nsplit][pairs][4] floats.  All compute-wave threads; the workgroup has no
// other item in the interval (the plan gives each workgroup at most one item when splits are used).
template <int G>
MBK_DEV void merge_slice(const Params &p, int j, int s, int gh, int hb, int nsplit, float *scr, uint32_t tag,
                         Ctl &ctl, StepCtx &sc) {
    const int hd = p.hd, npairs = gh * hd / 2;
    const int np = s < npairs ? (npairs - s + nsplit - 1) / nsplit : 0;
    cw_barrier(p, ctl, sc.gen);  // compute wave 0 is done with the wave partials in scr
    for (int i = threadIdx.x; i < nsplit * np; i += kCW * 64) {
        const int q = i / np, pi = i - q * np, v = s + pi * nsplit, h = (2 * v) / hd, e = 2 * v - h * hd;
        const uint32_t e0 = (uint32_t)(((j * p.max_splits + q) * G + hb + h) * (hd + 2));
        const uint32_t oa = (uint32_t)p.wl.part + 8u * (e0 + (uint32_t)hd), ob = (uint32_t)p.wl.part + 8u * (e0 + (uint32_t)e);
        u32x4 a, b;
        for (int it = 0;; ++it) {
            a = ldc16(p.ws, oa);
            b = ldc16(p.ws, ob);
            const bool ready = a.y == tag && a.w == tag && b.y == tag && b.w == tag;
            if (ready || it >= p.spin_limit || aborted(p, it)) {
                if (!ready && it >= p.spin_limit) set_error(p);
                break;
            }
            reread();
        }
        *(float4 *)(scr + 4 * i) = make_float4(__uint_as_float(a.x), __uint_as_float(a.z), __uint_as_float(b.x),
                                               __uint_as_float(b.z));
    }
    cw_barrier(p, ctl, sc.gen);
    for (int pi = threadIdx.x; pi < np; pi += kCW * 64) {
        const int v = s + pi * nsplit, h = (2 * v) / hd, e = 2 * v - h * hd;
        float mm = -INFINITY;
        for (int q = 0; q < nsplit; ++q) mm = fmaxf(mm, scr[4 * (q * np + pi)]);
        float ll = 0.f, a0 = 0.f, a1 = 0.f;
        for (int q = 0; q < nsplit; ++q) {
            const float *r = scr + 4 * (q * np + pi);
            const float c = r[0] == -INFINITY ? 0.f : __expf(r[0] - mm);  // a split without positions
            ll = fmaf(r[1], c, ll);
            a0 = fmaf(r[2], c, a0);
            a1 = fmaf(r[3], c, a1);
        }
        put2(p, p.wl.o, (j * G + hb + h) * hd + e, a0 / ll, a1 / ll, tag);
    }
}

// One attention item, for head size LP * 8 (LP lanes per position).
template <int G, int LP>
MBK_DEV void attention_task(const Params &p, const Interval &iv, int ivi, const Task &T, uint8_t *lds, Ctl &ctl,
                            RingPos &rp, StepCtx &sc) {
    constexpr int hd = LP * 8, PPW = 64 / LP;
    const int pos = sc.pos;
    const int lane = threadIdx.x & 63, cw = wave_id(), dl = lane & (LP - 1), slot = lane / LP;
    const AttnItem item = attn_item(T);
    const int j = item.j, s = item.s, h0 = item.h0, nh = item.nh;
    if (s >= sc.ss.nsplit) return;  // no allocations either
    const Range sp = split_range(sc.ss, s);
    const int nsplit = sc.ss.nsplit;
    const float *qkv = (const float *)(lds + p.lds_qkv + sc.in);
    const float *cur = qkv + G * hd;        // this step's key, then value
    // the queries as hi/lo bf16 pairs for the cached (bf16) keys: dot2 on the packed keys (this step's
    // key, in fp32, meets the fp32 queries, read again from LDS)
    u32x4 qh[G], ql[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        if (h >= nh) break;
        float v[8];
        load8f(qkv + h * hd + dl * 8, v);
        qh[h].x = to_bf16x2(v[0], v[1]); qh[h].y = to_bf16x2(v[2], v[3]);
        qh[h].z = to_bf16x2(v[4], v[5]); qh[h].w = to_bf16x2(v[6], v[7]);
        ql[h].x = to_bf16x2(v[0] - bf_lo(qh[h].x), v[1] - bf_hi(qh[h].x));
        ql[h].y = to_bf16x2(v[2] - bf_lo(qh[h].y), v[3] - bf_hi(qh[h].y));
        ql[h].z = to_bf16x2(v[4] - bf_lo(qh[h].z), v[5] - bf_hi(qh[h].z));
        ql[h].w = to_bf16x2(v[6] - bf_lo(qh[h].w), v[7] - bf_hi(qh[h].w));
    }
    float M[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        M[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }
    const uint8_t *ring = lds + p.lds_ring;
    const int na = n_allocs(p, iv, T, sc.ss);
    // cached positions, one ring piece at a time: each round a lane takes NB positions (blocks b,
    // b + kCW, ... of its wave), whose scores are independent of each other, and folds them into its
    // running state with one rescale
    constexpr int NB = G <= 4 ? 4 : (G <= 6 ? 2 : 1);
    for (int k = 0; k < na; ++k) {
        const Alloc A = task_alloc(p, iv, T, sc.ss, k);
        const uint8_t *kb = ring + ring_acquire(p, ctl, rp, A);
        const uint8_t *vb = kb + A.r1;
        const int nring = (int)(A.b0 / (uint32_t)(hd * 2));
        for (int b = cw; b * PPW < nring; b += kCW * NB) {
            u32x4 kw[NB], vw[NB];
            bool ok[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int t = (b + u * kCW) * PPW + slot;
                ok[u] = t < nring;
                const size_t at = (size_t)(ok[u] ? t : nring - 1) * hd * 2 + dl * 16;  // in the piece
                kw[u] = *(const u32x4 *)(kb + at);
                vw[u] = *(const u32x4 *)(vb + at);
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                if (h >= nh) break;
                float d[NB];
#pragma unroll
                for (int u = 0; u < NB; ++u) {
                    float x = 0.f;
                    x = dot2(kw[u].x, qh[h].x, x); x = dot2(kw[u].y, qh[h].y, x);
                    x = dot2(kw[u].z, qh[h].z, x); x = dot2(kw[u].w, qh[h].w, x);
                    x = dot2(kw[u].x, ql[h].x, x); x = dot2(kw[u].y, ql[h].y, x);
                    x = dot2(kw[u].z, ql[h].z, x); x = dot2(kw[u].w, ql[h].w, x);
                    d[u] = x;
                }
                float mn = M[h];
#pragma unroll
                for (int u = 0; u < NB; ++u) {
                    d[u] = ok[u] ? group_sum<LP>(d[u]) : -INFINITY;
                    mn = fmaxf(mn, d[u]);
                }
                // new maximum mn: what the lane holds is scaled by exp(M - mn), each position weighs
                // exp(d - mn); a lane that has seen no position yet keeps zeros (base 0 avoids -inf - -inf)
                const float base = mn == -INFINITY ? 0.f : mn;
                const float c = __expf(M[h] - base);
                float w[NB];
#pragma unroll
                for (int u = 0; u < NB; ++u) w[u] = __expf(d[u] - base);
                float ws = w[0];
#pragma unroll
                for (int u = 1; u < NB; ++u) ws += w[u];
                l[h] = fmaf(l[h], c, ws);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= c;
#pragma unroll
                for (int u = 0; u < NB; ++u) {
                    float vf[8];
                    unpack8(vw[u], vf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(w[u], vf[e], acc[h][e]);
                }
                M[h] = mn;
            }
        }
        ring_release(ctl, rp);
    }
    // the position appended this step (fp32 key and value in LDS, against the fp32 queries): slot 0 of
    // the last compute wave
    if (pos >= sp.t0 && pos < sp.t1 && cw == kCW - 1) {
        float kf[8], vf[8];
        load8f(cur + dl * 8, kf);
        load8f(cur + hd + dl * 8, vf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (h >= nh) break;
            float qf[8];
            load8f(qkv + h * hd + dl * 8, qf);
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d = fmaf(qf[e], kf[e], d);
            d = group_sum<LP>(d);
            if (slot == 0) {
                const float mn = fmaxf(M[h], d), c = __expf(M[h] - mn), w = __expf(d - mn);
                l[h] = fmaf(l[h], c, w);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(w, vf[e], acc[h][e] * c);
                M[h] = mn;
            }
        }
    }
    // wave partials {max, sum, -, -, acc[hd]} to LDS (the slots of the wave combined by the log-sum-exp
    // rule); compute wave 0 combines them
    const int stride = hd + 4;
    float *scr = (float *)(lds + p.lds_attn);  // [kCW][G][stride]
#pragma unroll
    for (int h = 0; h < G; ++h) {
        if (h >= nh) break;
        const float mw = slot_max<LP>(M[h]);
        const float c = M[h] == -INFINITY ? 0.f : __expf(M[h] - mw);  // a slot without positions adds nothing
        l[h] = slot_sum<LP>(l[h] * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = slot_sum<LP>(acc[h][e] * c);
        if (slot == 0) {
            float *r = scr + ((size_t)cw * G + h) * stride;
            if (dl == 0) {
                r[0] = mw;
                r[1] = l[h];
            }
            store8(r + 4 + dl * 8, acc[h]);
        }
    }
    cw_barrier(p, ctl, sc.gen);
    const uint32_t tag = tag_of(sc.tag0, ivi);
    if (cw == 0) {
        // log-sum-exp combination of the wave partials, one head dimension per lane (a wave without
        // positions has max -inf)
        for (int u = lane; u < nh * hd; u += 64) {
            const int h = u / hd, d = u % hd;
            float mw = -INFINITY;
            for (int w = 0; w < kCW; ++w) mw = fmaxf(mw, scr[((size_t)w * G + h) * stride]);
            float ll = 0.f, a = 0.f;
            for (int w = 0; w < kCW; ++w) {
                const float *r = scr + ((size_t)w * G + h) * stride;
                const float c = r[0] == -INFINITY ? 0.f : __expf(r[0] - mw);
                ll = fmaf(r[1], c, ll);
                a = fmaf(r[4 + d], c, a);
            }
            if (p.merge_in_o || (p.merge_dist && nsplit > 1)) {
                // tagged partial: entries [acc[hd] | max, sum] of (j, s, h)
                const int e0 = ((j * p.max_splits + s) * G + h0 + h) * (hd + 2);
                put(p, p.wl.part, e0 + d, a, tag);
                if (d == 0) put2(p, p.wl.part, e0 + hd, mw, ll, tag);
            } else if (nsplit == 1) {
                put(p, p.wl.o, (j * G + h0 + h) * hd + d, a / ll, tag);
            } else {
                // this split's partial: part[j][s][h][stride] = {max, sum, -, -, acc[hd]}
                const uint64_t pb = p.wl.part + ((uint64_t)(j * p.max_splits + s) * G + h0 + h) * stride * 4u;
                uint32_t *pw = ws_ptr<uint32_t>(p, pb);
                stc_u(pw + 4 + d, __float_as_uint(a));
                if (d == 0) {
                    stc_u(pw, __float_as_uint(mw));
                    stc_u(pw + 1, __float_as_uint(ll));
                }
            }
        }
    }
    if (nsplit > 1 && !p.merge_in_o && p.merge_dist) {
        // every split merges a slice of its group's outputs from the tagged partials of all splits
        // (a merge group is the query head of a single-head item, else the G heads of the KV head)
        merge_slice<G>(p, j, s, nh == 1 ? 1 : G, nh == 1 ? h0 : 0, nsplit, scr, tag, ctl, sc);
    } else if (nsplit > 1 && !p.merge_in_o) {
        // the last split to arrive (one atomic per split) merges the partials in split order, so the
        // result does not depend on arrival order.  A merge group is the query head of a single-head
        // item (gh = 1 head, counter j * G + h0), else the KV head (gh = G heads, counter j)
        const int gh = nh == 1 ? 1 : G, hb = nh == 1 ? h0 : 0, grp = nh == 1 ? j * G + h0 : j;
        if (threadIdx.x == 0) {
            __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are complete
            uint32_t *cnt = ws_ptr<uint32_t>(p, p.wl.merge_cnt + 256u * (uint32_t)grp);
            const bool last = atom_add(cnt, 1u) == (uint32_t)nsplit - 1u;
            if (last) {
                stc_u(cnt, 0u);
                __builtin_amdgcn_s_waitcnt(0);  // the reset lands before this group's output does
            }
            lds_st((uint32_t *)&ctl.last_s, last ? 1u : 0u);
        }
        cw_barrier(p, ctl, sc.gen);
        if (lds_ld((const uint32_t *)&ctl.last_s)) {
            // the group's partials into LDS: scr[(q * gh + h) * stride] for split q, head hb + h (the
            // scratch holds max_splits * G * stride floats)
            constexpr int c16 = (hd + 4) / 4;  // 16-byte chunks of one partial
            for (int idx = threadIdx.x; idx < nsplit * gh * c16; idx += kCW * 64) {
                const int qh = idx / c16, c = idx - qh * c16, q = qh / gh, h = qh - q * gh;
                const uint64_t src = p.wl.part + (((uint64_t)(j * p.max_splits + q) * G + hb + h) * stride + 4u * c) * 4u;
                *(u32x4 *)(scr + (size_t)qh * stride + 4 * c) = ldc16(p.ws, (uint32_t)src);
            }
            cw_barrier(p, ctl, sc.gen);
            for (int idx = 2 * threadIdx.x; idx < gh * hd; idx += 2 * kCW * 64) {
                const int h = idx / hd, e = idx % hd;
                // the largest split maximum first: then the splits' weights are independent of each other
                float mm = -INFINITY;
                for (int q = 0; q < nsplit; ++q) mm = fmaxf(mm, scr[((size_t)q * gh + h) * stride]);
                float ll = 0.f, a0 = 0.f, a1 = 0.f;
                for (int q = 0; q < nsplit; ++q) {
                    const float *r = scr + ((size_t)q * gh + h) * stride;
                    const float c = r[0] == -INFINITY ? 0.f : __expf(r[0] - mm);  // a split without positions
                    ll = fmaf(r[1], c, ll);
                    a0 = fmaf(r[4 + e], c, a0);
                    a1 = fmaf(r[5 + e], c, a1);
                }
                put2(p, p.wl.o, (j * G + hb + h) * hd + e, a0 / ll, a1 / ll, tag);
            }
        }
    }
    // the scratch is reused by the next item of the interval (a later interval's item comes after
    // that interval's input barrier)
    if (!(T.flags & TASK_LAST)) cw_barrier(p, ctl, sc.gen);
}

// ---- compute waves: the interval loop -----------------------------------------------------------------

MBK_DEV Task task_at(const Params &p, const uint8_t *lds, int k) {
    const int32_t *src = (const int32_t *)(lds + p.lds_tasks) + 4 * k;
    Task t;
    t.iv = __builtin_amdgcn_readfirstlane(src[0]);
    t.a = __builtin_amdgcn_readfirstlane(src[1]);
    t.n = __builtin_amdgcn_readfirstlane(src[2]);
    t.flags = __builtin_amdgcn_readfirstlane(src[3]);
    return t;
}

// The inputs of interval ivi (first task T) into the input block not read by
// the previous interval (with a single block, after the other compute waves
// are done with it), then the RMSNorm statistic.
template <int G>
MBK_DEV void interval_inputs(const Params &p, const Interval &iv, const Task &T, int ivi, uint8_t *lds, Ctl &ctl,
                             StepCtx &sc) {
    const int par = (int)(sc.nin & 1u);
    ++sc.nin;
    if (p.in_double) sc.in = par * p.in_bytes;
    else cw_barrier(p, ctl, sc.gen);
    float ss = 0.f;
    if (iv.op == OP_ATTN) attn_inputs<G>(p, T, ivi, lds, sc);
    else ss = gemv_inputs<G>(p, iv, T, ivi, lds, sc);
    ss = group_sum<64>(ss);
    if ((threadIdx.x & 63) == 0) ctl.ss[par][wave_id()] = ss;
    cw_barrier(p, ctl, sc.gen);
    stamp(p, lds, ivi, 1);
    sc.rnorm = 1.f;
    if (iv.op == OP_QKV || iv.op == OP_GATEUP || iv.op == OP_LMHEAD) {
        static_assert(kCW == 4, "one 16-byte read of the partial sums");
        const u32x4 s4 = lds_ld16(ctl.ss[par]);
        const float tot = (__uint_as_float(s4.x) + __uint_as_float(s4.y)) +
                          (__uint_as_float(s4.z) + __uint_as_float(s4.w));
        sc.rnorm = rsqrtf(tot * p.inv_h + p.eps);
    }
}

// Barrier mode: the workgroup's compute waves meet, then one thread takes
// part in the grid barrier that closes interval ivi.
MBK_DEV void interval_barrier(const Params &p, uint8_t *lds, Ctl &ctl, StepCtx &sc, int ivi) {
    // every compute store of this interval is complete before arrival
    __builtin_amdgcn_s_waitcnt(0);
    cw_barrier(p, ctl, sc.gen);
    if (threadIdx.x == 0 && !grid_barrier_thread(p, p.epoch_base + (uint32_t)(ivi - p.first_iv) + 1u))
        lds_st(&ctl.abort, 1u);
    cw_barrier(p, ctl, sc.gen);
    stamp(p, lds, ivi, 3);
}

// Compute waves: every interval of [first_iv, last_iv) in order; tasks [0, nt)
// of this workgroup in LDS.  The loops have no early exit (see cw_barrier);
// false only when the debug switch made this workgroup leave.
template <int G>
MBK_DEV bool compute(const Params &p0, uint8_t *lds, Ctl &ctl, int nt, StepCtx &sc) {
    RingPos rp;
    rp.cur = RingCursor{0u, 0u};
#pragma unroll
    for (int w = 0; w < kLW; ++w) rp.cum[w] = rp.seen[w] = 0;
    const int cw = wave_id();
    int k = 0;
    for (int ivi = p0.first_iv; ivi < p0.last_iv; ++ivi) {
        const Params &p = params_opaque();
        if ((int)blockIdx.x == p.skip_wg && ivi == p.skip_interval) return false;
        const int tiv = k < nt ? task_at(p, lds, k).iv : -1;
        if (tiv == ivi) {
            const Interval iv = interval_at(p, ivi);
            stamp(p, lds, ivi, 0);
            const uint32_t tag = tag_of(sc.tag0, ivi);
            if (iv.op == OP_ATTN) {
                // items of the interval, each with its own inputs (an item that is not the interval's
                // last ends with a compute-wave barrier)
                for (;;) {
                    const Task T = task_at(p, lds, k);
                    // splits beyond this step's split count have nothing to do (nor anything to load)
                    if (attn_item(T).s < sc.ss.nsplit) {
                        read_prog(ctl, rp.seen);
                        interval_inputs<G>(p, iv, T, ivi, lds, ctl, sc);
                        switch (p.hd_shift) {  // head size 16, 32, 64 or 128
                            case 4: attention_task<G, 2>(p, iv, ivi, T, lds, ctl, rp, sc); break;
                            case 5: attention_task<G, 4>(p, iv, ivi, T, lds, ctl, rp, sc); break;
                            case 6: attention_task<G, 8>(p, iv, ivi, T, lds, ctl, rp, sc); break;
                            default: attention_task<G, 16>(p, iv, ivi, T, lds, ctl, rp, sc); break;
                        }
                    }
                    ++k;
                    if (T.flags & TASK_LAST) break;
                }
            } else {
                Task T = task_at(p, lds, k);
                // the loader's progress is read while the inputs are polled: the weights of the first
                // task are usually complete by then
                read_prog(ctl, rp.seen);
                interval_inputs<G>(p, iv, T, ivi, lds, ctl, sc);
                const uint32_t tile_bytes = (uint32_t)iv.mat.tb;
                for (;;) {
                    if (T.iv != ivi) T = task_at(p, lds, k);  // further runs of the interval
                    const Alloc A = task_alloc(p, iv, T, sc.ss, 0);
                    const uint8_t *wt = lds + p.lds_ring + ring_acquire(p, ctl, rp, A);
                    for (int t = cw; t < T.n; t += kCW) gemv_tile_op(p, iv, lds, wt + (size_t)t * tile_bytes, T.a + t, sc, tag);
                    ring_release(ctl, rp);
                    ++k;
                    if (T.flags & TASK_LAST) break;
                    T.iv = -1;
                }
                if (iv.op == OP_LMHEAD) argmax_publish(p, iv, ctl, sc);
            }
            stamp(p, lds, ivi, 2);
        }
        if (p.barrier && ivi + 1 < p.last_iv) interval_barrier(p, lds, ctl, sc, ivi);
    }
    return true;
}

// ---- launch prologue -------------------------------------------------------------------------

// Copies this workgroup's tasks of [first_iv, last_iv) and this step's RoPE
// row into LDS and clears the control words.  Returns the number of tasks.
// All threads.
MBK_DEV int prologue(const Params &p, uint8_t *lds, Ctl &ctl, int pos) {
    const int32_t *ti = p.task_idx + (size_t)blockIdx.x * (p.n_intervals + 1);
    const int k0 = ti[p.first_iv], k1 = ti[p.last_iv];
    const int nt = min(k1 - k0, p.max_tasks);
    const u32x4 *ts = (const u32x4 *)(p.tasks + k0);
    u32x4 *td = (u32x4 *)(lds + p.lds_tasks);
    for (int i = threadIdx.x; i < nt; i += kThreads) td[i] = ts[i];
    const int half = p.hd / 2;
    float *rope = (float *)(lds + p.lds_rope);
    for (int i = threadIdx.x; i < 2 * half; i += kThreads) rope[i] = p.rope[(size_t)pos * 2 * half + i];
    if (p.trace) {
        // this workgroup's stamps of [first_iv, last_iv) start at zero; the stores are complete before
        // the barrier below, so no stamp can be overtaken by them
        for (int i = threadIdx.x; i < (p.last_iv - p.first_iv) * 4; i += kThreads)
            p.trace[((size_t)(p.first_iv + i / 4) * p.n_wg + blockIdx.x) * 4 + (i % 4)] = 0;
        __builtin_amdgcn_s_waitcnt(0);
    }
    if (threadIdx.x == 0) {
        for (int w = 0; w < kLW; ++w) ctl.prog[w] = 0;
        for (int w = 0; w < kCW; ++w) ctl.cons[w] = 0;
        ctl.bar = 0;
        ctl.abort = 0;
    }
    __syncthreads();
    return nt;
}

// The step body shared by both executors.
template <int G>
MBK_DEV void run_step(const Params &p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ Ctl ctl;
    const int pos = step_pos(p);
    const int nt = prologue(p, lds, ctl, pos);
    if (wave_id() >= kCW) {
        loader(p, lds, ctl, nt, pos);
    } else {
        StepCtx sc;
        sc.pos = pos;
        sc.ss = step_split(p, pos);
        sc.token = step_token(p);
        sc.tag0 = step_tag0(p);
        sc.rnorm = 1.f;
        sc.gen = 0;
        sc.best = 0;
        sc.blk0 = 0;
        sc.in = 0;
        sc.nin = 0;
        if (p.first_iv == 0 && blockIdx.x == 0 && threadIdx.x == 0 && !p.step_from_ws) {
            // this step's inputs, for launches that read them from the workspace
            uint32_t *ctrl = ws_ptr<uint32_t>(p, p.wl.ctrl);
            stc_u(ctrl + 3, (uint32_t)p.token);
            stc_u(ctrl + 4, (uint32_t)p.pos);
            stc_u(ctrl + 5, p.tag0);
        }
        if (!compute<G>(p, lds, ctl, nt, sc)) lds_st(&ctl.abort, 1u);
    }
}

}  // namespace mbk
