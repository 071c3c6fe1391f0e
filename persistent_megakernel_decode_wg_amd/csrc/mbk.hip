// mbk.hip -- libmbk: kernels and the C ABI declared in include/mbk.h.
//
// Executors (MegaBake article, section "How a model gets in": phases grouped
// into barrier intervals, a table-driven persistent loop that dispatches a
// body per phase row):
//   k_persistent  one launch (plain by default, cooperative on request), one
//                 workgroup per CU, walks the static interval table; intervals hand activations over as
//                 tagged entries (dataflow), or -- in barrier mode -- close
//                 with a counting grid barrier as in the article;
//   k_interval    the same bodies, one launch per interval (the ablation).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <cstdarg>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mbk.h"
#include "bodies.h"
#include "layout.h"
#include "prefill.h"

using namespace mbk;

// ---- kernels ----------------------------------------------------------------------------------------

// Both executors run the same step body (run_step): the persistent kernel
// over every interval of the step, the ablation kernel over one interval per
// launch.  Every workgroup leaves after its last interval or at its first
// failed (expired) wait; the debug switch skip_wg/skip_interval makes one
// workgroup leave early so that the others' waits expire.
template <int G>
__global__ __launch_bounds__(kThreads) void k_persistent(Params p) {
    run_step<G>(p);
}

// Params must stay the first kernel argument and reach the body unmodified:
// the compute waves read it from the kernel-argument segment (params_opaque).
// The ablation's host sets first_iv / last_iv to the launch's interval.
template <int G>
__global__ __launch_bounds__(kThreads) void k_interval(Params p) {
    run_step<G>(p);
}

// One instance per query-group size G (query heads per KV head).
typedef void (*persistent_fn)(Params);
typedef void (*interval_fn)(Params);
static const persistent_fn kPersistent[kMaxGqa] = {k_persistent<1>, k_persistent<2>, k_persistent<3>, k_persistent<4>,
                                                   k_persistent<5>, k_persistent<6>, k_persistent<7>, k_persistent<8>};
static const interval_fn kInterval[kMaxGqa] = {k_interval<1>, k_interval<2>, k_interval<3>, k_interval<4>,
                                               k_interval<5>, k_interval<6>, k_interval<7>, k_interval<8>};

__global__ __launch_bounds__(kThreads) void k_barrier_bench(Params p, int n) {
    for (int i = 0; i < n; ++i)
        if (!grid_barrier(p, p.epoch_base + (uint32_t)i + 1u)) return;
}

// Grid-barrier validation (the counting barrier of the article's executor): in round i every workgroup
// writes i into its epoch slot, passes the barrier of epoch epoch_base + i, then reads every workgroup's
// slot, which must hold at least i (the barrier orders every write of round i before every read after it).
// The first failed check (lowest round) is recorded in res[0..3] = {round, reader, writer, value read};
// no workgroup leaves a round early, so every barrier still completes.  A barrier that times out (the
// bounded wait, reported through the error word) ends the workgroup's rounds.
__global__ __launch_bounds__(kThreads) void k_barrier_stress(Params p, int n, uint32_t *res, uint32_t *slots) {
    if ((int)blockIdx.x == p.skip_wg) return;   // test hook: this workgroup never arrives
    for (int i = 1; i <= n; ++i) {
        if (threadIdx.x == 0) stc_u(slots + blockIdx.x, (uint32_t)i);
        if (!grid_barrier(p, p.epoch_base + (uint32_t)i)) return;
        for (int w = threadIdx.x; w < p.n_wg; w += kThreads) {
            const uint32_t v = ldc_u(slots + w);
            if (v < (uint32_t)i) {
                const uint32_t old = atomicMin(res, (uint32_t)i);
                if (old > (uint32_t)i) {
                    stc_u(res + 1, blockIdx.x);
                    stc_u(res + 2, (uint32_t)w);
                    stc_u(res + 3, v);
                }
            }
        }
    }
}

// Packer: one thread per 16-byte chunk of the packed matrix.
__global__ void k_pack(uint8_t *dst, MatGeom g, const uint16_t *s0, const uint16_t *s1, const uint16_t *s2, int hd,
                       int nq_rows, int nkv_rows) {
    const uint64_t n = (uint64_t)g.ntiles * g.IT * 64u;
    for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n; c += (uint64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(c % 64u);
        const uint64_t rest = c / 64u;
        const int it = (int)(rest % (uint64_t)g.IT);
        const int64_t t = (int64_t)(rest / (uint64_t)g.IT);
        const int64_t prow = t * g.RT + lane / g.L;
        const int kg = (lane % g.L) + it * g.L;
        u32x4 v = {0u, 0u, 0u, 0u};  // rows past the matrix and padding groups are zero
        if (prow < g.rows && kg < g.K / 8) {
            RowSrc s = packed_row_source(g.kind, (int)prow, hd, nq_rows, nkv_rows);
            const uint16_t *src = s.which == 0 ? s0 : (s.which == 1 ? s1 : s2);
            v = *(const u32x4 *)(src + (uint64_t)s.row * g.K + (uint64_t)kg * 8u);
        }
        *(u32x4 *)(dst + chunk_offset(g, t, it, lane)) = v;
    }
}

// OCP E4M3 code of a finite x with |x| <= 448, rounded to nearest, ties to even (sign kept, zero
// included).  Below 2^-6 the values are the multiples of 2^-9 (the subnormals; 8 * 2^-9 is the smallest
// normal, code 8); above, the fp32 mantissa is rounded to 3 bits and the exponent rebiased from 127 to 7.
__device__ uint32_t e4m3_rne(float x) {
    const uint32_t b = __float_as_uint(x), s = (b >> 24) & 0x80u, a = b & 0x7fffffffu;
    if (a < 0x3c800000u) return s | (uint32_t)rintf(__uint_as_float(a) * 512.0f);
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) & ~0xfffffu;
    return s | ((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));
}

// Scale 2^e of an fp8 row with largest magnitude amax: e the smallest integer >= -126 with
// amax / 2^e <= 448 = 1.75 * 2^8 (1 for a zero row).  For amax = 1.m * 2^E: e = E - 8 when 1.m <= 1.75,
// else E - 7.
__device__ float fp8_row_scale(float amax) {
    const uint32_t b = __float_as_uint(amax);
    if (b == 0u) return 1.0f;
    const int E = (int)(b >> 23) - 127;
    int e = (b & 0x7fffffu) <= 0x600000u ? E - 8 : E - 7;
    if ((b >> 23) == 0u || e < -126) e = -126;
    return __uint_as_float((uint32_t)(e + 127) << 23);
}

MBK_DEV const uint16_t *source_row(const MatGeom &g, int64_t prow, const uint16_t *s0, const uint16_t *s1,
                                   const uint16_t *s2, int hd, int nq_rows, int nkv_rows) {
    const RowSrc s = packed_row_source(g.kind, (int)prow, hd, nq_rows, nkv_rows);
    return (s.which == 0 ? s0 : (s.which == 1 ? s1 : s2)) + (uint64_t)s.row * g.K;
}

// Scale blocks of an fp8 matrix: one thread per fp32 slot (the scale of a row, or zero padding).
__global__ void k_pack_scale(uint8_t *dst, MatGeom g, const uint16_t *s0, const uint16_t *s1, const uint16_t *s2,
                             int hd, int nq_rows, int nkv_rows) {
    const int per = (g.tb - g.IT * 1024) / 4;
    const uint64_t n = (uint64_t)g.ntiles * per;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x) {
        const int64_t t = (int64_t)(i / (uint64_t)per);
        const int slot = (int)(i % (uint64_t)per);
        const int64_t prow = t * g.RT + slot;
        float v = 0.f;
        if (slot < g.RT && prow < g.rows) {
            const uint16_t *src = source_row(g, prow, s0, s1, s2, hd, nq_rows, nkv_rows);
            float amax = 0.f;
            for (int k = 0; k < g.K; ++k) amax = fmaxf(amax, fabsf(__uint_as_float((uint32_t)src[k] << 16)));
            v = fp8_row_scale(amax);
        }
        *(float *)(dst + g.off + (uint64_t)t * g.tb + (uint64_t)g.IT * 1024u + (uint64_t)slot * 4u) = v;
    }
}

// Codes of an fp8 matrix (after k_pack_scale): one thread per 16-byte chunk of 16 codes, each the bf16
// weight divided by its row's scale (exactly: a power of two) and rounded by e4m3_rne.
__global__ void k_pack_fp8(uint8_t *dst, MatGeom g, const uint16_t *s0, const uint16_t *s1, const uint16_t *s2, int hd,
                           int nq_rows, int nkv_rows) {
    const uint64_t n = (uint64_t)g.ntiles * g.IT * 64u;
    for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n; c += (uint64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(c % 64u);
        const uint64_t rest = c / 64u;
        const int it = (int)(rest % (uint64_t)g.IT);
        const int64_t t = (int64_t)(rest / (uint64_t)g.IT);
        const int64_t prow = t * g.RT + lane / g.L;
        const int kg = (lane % g.L) + it * g.L;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (prow < g.rows && kg < g.K / 16) {
            const uint16_t *src = source_row(g, prow, s0, s1, s2, hd, nq_rows, nkv_rows) + (uint64_t)kg * 16u;
            const uint32_t sb = __float_as_uint(*(const float *)(dst + row_scale_offset(g, prow)));
            const float inv = __uint_as_float((254u << 23) - (sb & 0x7f800000u));   // 2^-e
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                w[q] = 0u;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    w[q] |= e4m3_rne(__uint_as_float((uint32_t)src[4 * q + j] << 16) * inv) << (8 * j);
            }
            v = (u32x4){w[0], w[1], w[2], w[3]};
        }
        *(u32x4 *)(dst + chunk_offset(g, t, it, lane)) = v;
    }
}

// ---- the workspace of callers that cannot allocate ----------------------------------------------------
// mbk_decode_step_static runs the step with this array as its workspace.  Every device holds its own
// copy until the process ends; host code reaches it only through the device address that
// hipGetSymbolAddress returns for the current device (the array's name is a host-side stand-in).
constexpr size_t kStaticScratchBytes = 512u << 10;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// Clears n bytes (a multiple of 16) at p.  A kernel rather than a memset node, so a caller may capture
// the call into a graph.
__global__ void k_zero16(uint8_t *p, uint64_t n) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x * 16u;
    for (uint64_t i = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) * 16u; i < n; i += stride)
        *(u32x4 *)(p + i) = (u32x4){0u, 0u, 0u, 0u};
}

// ---- host side --------------------------------------------------------------------------------------

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

#define HIPCHK(call)                                                                              \
    do {                                                                                          \
        hipError_t e_ = (call);                                                                   \
        if (e_ != hipSuccess) return fail(MBK_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
    } while (0)

struct LayerPlan {
    MatGeom qkv, o, gu, down;
    uint64_t attn_norm, mlp_norm, bias;  // bias = ~0 when absent
};

struct Plan {
    std::vector<LayerPlan> layers;
    MatGeom embed;   // bf16 table of the embedding row gathers
    MatGeom lmhead;  // vocabulary projection: the embedding itself (bf16), or its fp8 copy
    uint64_t final_norm = 0, rope = 0, table = 0, tasks = 0, task_idx = 0, total = 0;
    std::vector<Interval> iv;
    std::vector<Task> task_list;       // all workgroups' tasks, workgroup-major
    std::vector<int32_t> task_index;   // [n_wg][n_iv + 1]
    int max_splits = 1, piece_pos = 1, max_tasks = 0, in_bytes = 0, in_double = 0, attn_hpi = 1;
    // LDS layout (bytes of the dynamic area)
    int lds_tasks = 0, lds_rope = 0, lds_qkv = 0, lds_bias = 0, lds_xs = 0,
        lds_xres = 0, lds_attn = 0, lds_ring = 0, ring_bytes = 0;
    size_t lds_bytes = 0;
    WsLayout ws{};
};

// State of one device's static scratch, shared by every handle that runs mbk_decode_step_static there.
struct StaticScratch {
    uint8_t *ptr = nullptr;   // device address of this device's `scratch`
    uint32_t next_tag = 1;    // first tag of the next step run on it (tags never repeat until it is cleared)
    uint32_t epoch = 0;       // grid barriers completed on it
    bool clean = false;       // cleared since first use and since the last error mbk_check saw
};
std::mutex g_static_mu;
std::vector<StaticScratch> g_static;   // by device index

}  // namespace

struct mbk_model {
    mbk_config c;
    int n_wg = 0;
    int device = -1;
    bool planned = false;
    Plan plan;
    std::vector<float> rope_host;
    uint8_t *blob = nullptr;
    uint16_t *kv = nullptr;
    uint8_t *ws = nullptr;
    uint32_t epoch = 0;   // grid barriers completed on the bound workspace
    uint32_t seq = 0;     // decode steps run on the bound workspace (their tags: seq * intervals + 1 on)
    int32_t sync_mode = MBK_SYNC_DATAFLOW;
    int32_t launch_mode = MBK_LAUNCH_PLAIN;
    int32_t spin_limit = 1 << 22, skip_wg = -1, skip_interval = -1;
    int32_t attn_min_chunk = 128;
    int32_t n_wg_set = 0;        // mbk_set_workgroups (0: every compute unit)
    int32_t attn_items_set = 0;  // mbk_set_attention_items (0: automatic)
    int32_t weight_fmt = 0;      // mbk_set_weight_format: FMT_BF16 or FMT_FP8
    bool kernels_ready = false;
    uint64_t *trace = nullptr;
    // graph replay of the ablation
    hipGraph_t graph = nullptr;
    hipGraphExec_t gexec = nullptr;
    hipGraphNode_t node0 = nullptr;
    float *g_logits = nullptr;
    int32_t *g_argmax = nullptr;
    int static_dev = -1;   // device whose static scratch this handle last stepped on (mbk_check reads it)
};

namespace {

// An operator with fewer tiles than workgroups leaves workgroups idle while
// each tile is one wave's chain of IT dependent steps.  Such an operator, if
// its rows need no pairing, takes one row per tile (L = 64: the fewest steps,
// up to 4 tiles per workgroup, one per compute wave) over inputs padded with
// zero groups to a multiple of 64, when the padding stays within 15 % of the
// bytes.  (Measured on MI355X: one-row tiles help where they turn idle
// workgroups into busy waves, e.g. the Qwen2-0.5B output projection; tiles of
// 2-4 rows over more workgroups do not.)
MatGeom make_geom(uint64_t &cursor, int rows, int K, bool pairs, int kind, int n_wg, int fmt) {
    MatGeom g{};
    g.fmt = fmt;
    g.gv = fmt == FMT_FP8 ? 16 : 8;
    choose_lanes(K, g.gv, pairs, &g.L, &g.RT);
    const int kg = K / g.gv;
    int kgp = kg;
    const int kg64 = (kg + 63) / 64 * 64;
    if (!pairs && g.L < 64 && (rows + g.RT - 1) / g.RT < n_wg && (int64_t)kg64 * 100 <= (int64_t)kg * 115) {
        g.L = 64;
        g.RT = 1;
        kgp = kg64;
    }
    // bf16 rows of 2,048 inputs (4 KiB) go two to a tile where there are rows enough for every workgroup: each
    // tile's reduction and epilogue then serve two rows
    if (!pairs && fmt == FMT_BF16 && g.L == 64 && kg == 256 && (rows + 1) / 2 >= n_wg) {
        g.L = 32;
        g.RT = 2;
    }
    g.K = K;
    g.IT = kgp / g.L;
    g.rows = rows;
    g.ntiles = (rows + g.RT - 1) / g.RT;
    g.kind = kind;
    g.lrt = 0;
    while ((1 << g.lrt) < g.RT) ++g.lrt;
    g.tb = tile_bytes_of(fmt, g.IT, g.RT);
    g.off = cursor;
    cursor = align256(cursor + (uint64_t)g.ntiles * g.tb);
    return g;
}

Interval gemv_interval(int op, int layer, const MatGeom &g, uint64_t norm, uint64_t bias, int x_src) {
    Interval v{};
    v.op = op;
    v.layer = layer;
    v.n_items = g.ntiles;
    v.x_src = x_src;
    v.mat = g;
    v.norm_off = norm;
    v.bias_off = bias;
    return v;
}

// Workgroup count: the value set with mbk_set_workgroups, else the current
// device's compute units.
int ensure_device(mbk_model *m) {
    if (m->n_wg > 0) return MBK_OK;
    if (m->n_wg_set > 0) {
        m->n_wg = m->n_wg_set;
        return MBK_OK;
    }
    HIPCHK(hipGetDevice(&m->device));
    int cus = 0;
    HIPCHK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, m->device));
    if (cus <= 0) return fail(MBK_ERR_HIP, "device reports %d compute units", cus);
    m->n_wg = cus;
    return MBK_OK;
}

// Launch attributes of the kernels for this plan (once per handle, on the current device).
int ensure_kernels(mbk_model *m) {
    if (m->kernels_ready) return MBK_OK;
    int cus = 0, dev = 0;
    HIPCHK(hipGetDevice(&dev));
    HIPCHK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    if (m->n_wg > cus)
        return fail(MBK_ERR_UNSUPPORTED, "%d workgroups requested but the device has %d compute units", m->n_wg, cus);
    const int G = m->c.n_heads / m->c.n_kv_heads;
    const int lds = (int)m->plan.lds_bytes;
    HIPCHK(hipFuncSetAttribute((const void *)kPersistent[G - 1], hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    HIPCHK(hipFuncSetAttribute((const void *)kInterval[G - 1], hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    // a plain launch relies on one resident workgroup per compute unit
    int per_cu = 0;
    HIPCHK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)kPersistent[G - 1], kThreads, (size_t)lds));
    if (per_cu < 1) return fail(MBK_ERR_UNSUPPORTED, "the persistent kernel does not fit on a compute unit");
    m->kernels_ready = true;
    return MBK_OK;
}

constexpr size_t kLdsMax = 160 * 1024;
constexpr size_t kLdsStatic = 512;      // Ctl and the other static LDS words of the kernels
constexpr int kMinRing = 16 * 1024;
constexpr int kPiecePos = 128;          // most cached positions per attention piece
constexpr int kMinSplitPos = 32;        // fewest positions per attention split the plan provides for

size_t a16(size_t v) { return (v + 15) / 16 * 16; }

// Builds the packed-blob layout, the interval table, every workgroup's task
// list and the LDS layout.  Returns an empty string or the reason the shape
// cannot be planned.
std::string build_plan(mbk_model *m) {
    const mbk_config &c = m->c;
    Plan &P = m->plan;
    const int n_wg = m->n_wg;
    const int hd = c.head_dim, Q = c.n_heads * hd, KV = c.n_kv_heads * hd, G = c.n_heads / c.n_kv_heads;
    if (m->weight_fmt == FMT_FP8 && (c.hidden % 16 || Q % 16 || c.intermediate % 16))
        return "fp8 weights need hidden, heads*head_dim and intermediate to be multiples of 16";
    uint64_t cur = 0;
    P.layers.resize(c.n_layers);
    for (int l = 0; l < c.n_layers; ++l) {
        LayerPlan &L = P.layers[l];
        const int f = m->weight_fmt;
        L.qkv = make_geom(cur, Q + 2 * KV, c.hidden, true, MAT_QKV, n_wg, f);
        L.o = make_geom(cur, c.hidden, Q, false, MAT_PLAIN, n_wg, f);
        L.gu = make_geom(cur, 2 * c.intermediate, c.hidden, true, MAT_GATEUP, n_wg, f);
        L.down = make_geom(cur, c.hidden, c.intermediate, false, MAT_PLAIN, n_wg, f);
        L.attn_norm = cur;
        cur = align256(cur + 2u * c.hidden);
        L.mlp_norm = cur;
        cur = align256(cur + 2u * c.hidden);
        L.bias = ~(uint64_t)0;
        if (c.qkv_bias) {
            L.bias = cur;
            cur = align256(cur + 2u * (Q + 2 * KV));
        }
    }
    P.embed = make_geom(cur, c.vocab, c.hidden, false, MAT_PLAIN, n_wg, FMT_BF16);
    P.lmhead = m->weight_fmt == FMT_FP8 ? make_geom(cur, c.vocab, c.hidden, false, MAT_PLAIN, n_wg, FMT_FP8) : P.embed;
    P.final_norm = cur;
    cur = align256(cur + 2u * c.hidden);
    P.rope = cur;
    cur = align256(cur + (uint64_t)c.kv_capacity * (hd / 2) * 8u);

    // attention splits: enough items to reach the CUs, and every partial of
    // one KV head fits the LDS merge scratch
    const int stride = hd + 4;
    const size_t merge_budget = 16 * 1024;
    // attention items: one per query head unless there are more query heads than workgroups (the G
    // items of a KV head then read its keys and values G times, mostly from the caches, but each
    // item's chain of dependent steps is G times shorter), else the query heads of a KV head packed
    // so each key and value is read once; mbk_set_attention_items overrides the choice
    P.attn_hpi = m->attn_items_set ? m->attn_items_set : (c.n_heads <= n_wg ? 1 : G);
    const int item_heads = P.attn_hpi == 1 ? c.n_heads : c.n_kv_heads;
    int ms = std::max(1, n_wg / item_heads);
    ms = std::min<int>(ms, (int)(merge_budget / ((size_t)G * stride * 4)));
    // splits shorter than kMinSplitPos positions are never useful: a short cache needs few
    ms = std::min(ms, (c.kv_capacity + kMinSplitPos - 1) / kMinSplitPos);
    ms = std::max(1, std::min(ms, 64));
    P.max_splits = ms;

    // intervals: participants rotate so that successive intervals start on different workgroups
    const uint64_t none = ~(uint64_t)0;
    P.iv.clear();
    for (int l = 0; l < c.n_layers; ++l) {
        const LayerPlan &L = P.layers[l];
        const int base = 5 * l, prev_down = l == 0 ? -1 : base - 1;
        P.iv.push_back(gemv_interval(OP_QKV, l, L.qkv, L.attn_norm, L.bias, prev_down));
        Interval a{};
        a.op = OP_ATTN;
        a.layer = l;
        a.n_items = item_heads * ms;
        a.x_src = -1;
        a.norm_off = a.bias_off = none;
        P.iv.push_back(a);
        P.iv.push_back(gemv_interval(OP_O, l, L.o, none, none, prev_down));
        P.iv.push_back(gemv_interval(OP_GATEUP, l, L.gu, L.mlp_norm, none, base + 2));
        P.iv.push_back(gemv_interval(OP_DOWN, l, L.down, none, none, base + 2));
    }
    P.iv.push_back(gemv_interval(OP_LMHEAD, -1, P.lmhead, P.final_norm, none, 5 * c.n_layers - 1));
    const int n_iv = (int)P.iv.size();
    for (const Interval &v : P.iv)
        if (v.n_items >= (1 << 23)) return "too many tiles in one operator";
    int rot = 0;
    for (Interval &v : P.iv) {
        v.nwg = std::min(n_wg, v.n_items);
        v.wg0 = rot;
        rot = (rot + v.nwg) % n_wg;
    }

    // LDS layout (the ring takes what is left)
    int max_rows = 1;
    for (const Interval &v : P.iv)
        if (v.op == OP_O || v.op == OP_DOWN)
            for (int k = 0; k < v.nwg; ++k)
                max_rows = std::max(max_rows, (block_begin(v.n_items, k + 1, v.nwg) - block_begin(v.n_items, k, v.nwg)) * v.mat.RT);
    int kmax = 8;  // longest (padded) GEMV input
    for (const Interval &v : P.iv)
        if (v.op != OP_ATTN) kmax = std::max(kmax, v.mat.IT * v.mat.L * v.mat.gv);
    size_t off = 0;
    const size_t task_slot = off;
    // tasks are laid out below, once their count is known; reserve after the fixed parts
    P.lds_rope = 0;
    size_t fixed = 0;
    fixed += a16((size_t)4 * hd);                                  // RoPE row
    fixed += a16((size_t)(G + 2) * hd * 4);                        // attention inputs
    fixed += c.qkv_bias ? a16((size_t)(Q + 2 * KV) * 4) : 0;       // Q/K/V bias
    fixed += a16((size_t)kmax * 4);                                // GEMV input (hi/lo pairs)
    fixed += a16((size_t)max_rows * 4);                            // residual rows
    fixed += a16((size_t)std::max(kCW, ms) * G * stride * 4);      // attention merge scratch
    // input block [attention inputs | bias | GEMV input | residual rows]; a second copy lets an
    // interval's inputs load while other compute waves still read the previous interval's
    const size_t in_block = a16((size_t)(G + 2) * hd * 4) + (c.qkv_bias ? a16((size_t)(Q + 2 * KV) * 4) : 0) +
                            a16((size_t)kmax * 4) + a16((size_t)max_rows * 4);
    {
        // the second copy costs ring space: it is kept only while it is small.  Where the weights per
        // workgroup and interval exceed the ring (streaming-bound shapes) the ring is worth more: the
        // bytes in flight per workgroup are bounded by its free part.
        // fixed holds one copy already: left is what a second copy leaves.
        const size_t left = kLdsMax - kLdsStatic - task_slot - fixed - in_block;
        P.in_double = left > (size_t)64 * 16 + 64 * 1024 && in_block <= 16 * 1024 ? 1 : 0;
        if (P.in_double) fixed += in_block;
    }

    // tile runs of at most a third of the ring: first size the ring assuming a task
    // list of 64 entries per workgroup, then build the lists and shrink the ring
    // to what the lists leave.
    size_t max_tile = 0;
    for (const Interval &v : P.iv)
        if (v.op != OP_ATTN) max_tile = std::max(max_tile, (size_t)v.mat.tb);
    auto build_tasks = [&](size_t ring) {
        // a run takes at most a third of the ring (the loader then has two runs' room while one is computed:
        // the SmolLM-1.7B down projection's 16 KiB tiles go two to a run rather than three)
        const size_t max_alloc = ring / 3;
        P.task_list.clear();
        P.task_index.assign((size_t)n_wg * (n_iv + 1), 0);
        int max_tasks = 0;
        for (int w = 0; w < n_wg; ++w) {
            const int start = (int)P.task_list.size();
            for (int i = 0; i < n_iv; ++i) {
                P.task_index[(size_t)w * (n_iv + 1) + i] = (int)P.task_list.size();
                const Interval &v = P.iv[i];
                const int k = participant(v, w, n_wg);
                if (k < 0) continue;
                const size_t first = P.task_list.size();
                if (v.op == OP_ATTN) {
                    for (int it = k; it < v.n_items; it += v.nwg)
                        P.task_list.push_back(Task{i, it, attn_task_item(it, P.max_splits, G, P.attn_hpi), 0});
                } else {
                    const int b0 = block_begin(v.n_items, k, v.nwg), b1 = block_begin(v.n_items, k + 1, v.nwg);
                    // a block longer than one run goes in runs of whole rounds of the compute waves (a
                    // multiple of kCW tiles, at least one round) of at most a third of the ring: the ring
                    // then holds three runs or more, so the bytes in flight are what the run being
                    // computed leaves free, and each run still gives every compute wave several tiles
                    int per = std::max<int>(1, (int)(max_alloc / (size_t)v.mat.tb));
                    if (per >= kCW && b1 - b0 > per)
                        per = std::max<int>(kCW, (int)(ring / 3 / ((size_t)kCW * v.mat.tb)) * kCW);
                    for (int t = b0; t < b1; t += per)
                        P.task_list.push_back(Task{i, t, std::min(per, b1 - t), b1 << 8});
                }
                if (P.task_list.size() > first) {
                    P.task_list[first].flags |= TASK_FIRST;
                    P.task_list.back().flags |= TASK_LAST;
                }
            }
            P.task_index[(size_t)w * (n_iv + 1) + n_iv] = (int)P.task_list.size();
            max_tasks = std::max(max_tasks, (int)P.task_list.size() - start);
        }
        P.max_tasks = max_tasks;
    };
    const size_t avail0 = kLdsMax - kLdsStatic - task_slot - fixed;
    size_t ring = avail0 > (size_t)64 * 16 ? (avail0 - 64 * 16) / kChunk * kChunk : 0;
    for (int iter = 0; iter < 4; ++iter) {
        if (ring < (size_t)kMinRing || ring < 3 * max_tile) break;
        build_tasks(ring);
        const size_t need = task_slot + a16((size_t)P.max_tasks * 16) + fixed;
        if (need + kLdsStatic + ring <= kLdsMax) break;
        ring = need + kLdsStatic < kLdsMax ? (kLdsMax - kLdsStatic - need) / kChunk * kChunk : 0;
    }
    if (ring < (size_t)kMinRing || ring < 3 * max_tile)
        return "not enough LDS for the weight ring (" + std::to_string(ring) + " bytes)";
    build_tasks(ring);
    off = task_slot;
    P.lds_tasks = (int)off; off = a16(off + (size_t)P.max_tasks * 16);
    P.lds_rope = (int)off; off = a16(off + (size_t)4 * hd);
    P.lds_qkv = (int)off; off = a16(off + (size_t)(G + 2) * hd * 4);
    P.lds_bias = (int)off; off = c.qkv_bias ? a16(off + (size_t)(Q + 2 * KV) * 4) : off;
    P.lds_xs = (int)off; off = a16(off + (size_t)kmax * 4);
    P.lds_xres = (int)off; off = a16(off + (size_t)max_rows * 4);
    P.in_bytes = (int)(off - (size_t)P.lds_qkv);
    if (P.in_double) off += P.in_bytes;
    P.lds_attn = (int)off; off = a16(off + (size_t)std::max(kCW, ms) * G * stride * 4);
    off = (off + kChunk - 1) / kChunk * kChunk;
    P.lds_ring = (int)off;
    if (off + ring + kLdsStatic > kLdsMax) ring = (kLdsMax - kLdsStatic - off) / kChunk * kChunk;
    if (ring < (size_t)kMinRing || ring < 3 * max_tile) return "not enough LDS for the weight ring";
    // task runs were cut for the ring size used by build_tasks; re-cut if the ring shrank
    build_tasks(ring);
    if (P.lds_tasks + (size_t)P.max_tasks * 16 > (size_t)P.lds_rope) return "task list does not fit its LDS slot";
    P.ring_bytes = (int)ring;
    P.lds_bytes = off + ring;
    // attention pieces: at most a third of the ring, keys and values each rounded up to whole chunks; where
    // every split holds at most 2 kPiecePos positions, up to that many in one piece of at most 60 % of the ring
    // (one piece per split: its bookkeeping once)
    const int longest = std::max((c.kv_capacity + P.max_splits - 1) / P.max_splits, (int)m->attn_min_chunk);
    const bool one_piece = longest <= 2 * kPiecePos;
    P.piece_pos = std::min(one_piece ? 2 * kPiecePos : kPiecePos,
                           (int)(((one_piece ? ring * 6 / 10 : ring / 3) / 2) / kChunk * kChunk / ((size_t)hd * 2)));
    if (P.piece_pos < 1) return "attention piece too small";
    while (P.piece_pos & (P.piece_pos - 1)) P.piece_pos &= P.piece_pos - 1;  // a power of two

    P.table = cur;
    cur = align256(cur + P.iv.size() * sizeof(Interval));
    P.tasks = cur;
    cur = align256(cur + P.task_list.size() * sizeof(Task));
    P.task_idx = cur;
    cur = align256(cur + P.task_index.size() * sizeof(int32_t));
    P.total = cur;

    // workspace
    WsLayout &W = P.ws;
    uint64_t w = 0;
    W.ctrl = w; w += 256;
    W.argkey = w; w += 256;
    W.bar_global = w; w += 256;
    W.bar_group = w; w += 256 * kGroups;
    W.bar_rel = w; w += 256 * kGroups;
    W.merge_cnt = w; w += 256u * c.n_heads;   // one line per merge group (query head or KV head)
    // tagged activations: 8 bytes per entry
    W.x = w; w = align256(w + 8u * c.hidden);
    W.q = w; w = align256(w + 8u * Q);
    W.k = w; w = align256(w + 8u * KV);
    W.v = w; w = align256(w + 8u * KV);
    W.o = w; w = align256(w + 8u * Q);
    W.a = w; w = align256(w + 8u * c.intermediate);
    // attention partials: fp32 [nkv][ms][G][hd + 4] for the last-arriver merge, or tagged
    // 8-byte entries [nkv][ms][G][hd + 2] for the merge in the output projection
    W.part = w;
    w = align256(w + std::max<uint64_t>(4u * (uint64_t)c.n_kv_heads * ms * G * stride,
                                        8u * (uint64_t)c.n_kv_heads * ms * G * (hd + 2)));
    W.stress = w;
    w = align256(w + 16u + 4u * (uint64_t)n_wg);
    W.total = w;

    // RoPE table: angle pos * theta^(-2i/hd), evaluated in double, stored fp32
    m->rope_host.assign((size_t)c.kv_capacity * (hd / 2) * 2, 0.f);
    for (int pos = 0; pos < c.kv_capacity; ++pos)
        for (int i = 0; i < hd / 2; ++i) {
            const double ang = (double)pos * std::pow((double)c.rope_theta, -2.0 * i / (double)hd);
            m->rope_host[((size_t)pos * (hd / 2) + i) * 2 + 0] = (float)std::cos(ang);
            m->rope_host[((size_t)pos * (hd / 2) + i) * 2 + 1] = (float)std::sin(ang);
        }
    m->planned = true;
    return "";
}

int ensure_plan(mbk_model *m) {
    if (m->planned) return MBK_OK;
    int rc = ensure_device(m);
    if (rc) return rc;
    const std::string why = build_plan(m);
    if (!why.empty()) return fail(MBK_ERR_UNSUPPORTED, "%s", why.c_str());
    const size_t lds = m->plan.lds_bytes;
    if (lds + kLdsStatic > kLdsMax) return fail(MBK_ERR_UNSUPPORTED, "needs %zu bytes of LDS", lds);
    return MBK_OK;
}

// Next step number on the bound workspace: its tags seq * n_intervals + 1 + i
// must stay below 2^32.
uint32_t next_seq(mbk_model *m) {
    const uint32_t n = (uint32_t)m->plan.iv.size();
    m->seq = (m->seq + 1u >= 0xffffffffu / n - 1u) ? 1u : m->seq + 1u;
    return m->seq;
}

Params make_params(const mbk_model *m, int32_t token, int32_t pos, float *logits, int32_t *argmax) {
    const mbk_config &c = m->c;
    const Plan &P = m->plan;
    Params p{};
    p.blob = m->blob;
    p.iv = (const Interval *)(m->blob + P.table);
    p.tasks = (const Task *)(m->blob + P.tasks);
    p.task_idx = (const int32_t *)(m->blob + P.task_idx);
    p.kv = m->kv;
    p.ws = m->ws;
    p.wl = P.ws;
    p.logits = logits;
    p.argmax_out = argmax;
    p.rope = (const float *)(m->blob + P.rope);
    p.trace = m->trace;
    p.embed = P.embed;
    p.n_wg = m->n_wg;
    p.n_intervals = (int)P.iv.size();
    p.H = c.hidden;
    p.nq = c.n_heads;
    p.nkv = c.n_kv_heads;
    p.hd = c.head_dim;
    p.I = c.intermediate;
    p.V = c.vocab;
    p.S = c.kv_capacity;
    p.NL = c.n_layers;
    p.max_splits = P.max_splits;
    p.gqa = c.n_heads / c.n_kv_heads;
    p.attn_min_chunk = m->attn_min_chunk;
    {
        // the output projection merges the split partials itself when they are few: every one of
        // its workgroups polls nq * splits * (hd + 2) tagged entries
        const int splits = std::min(P.max_splits, (c.kv_capacity + m->attn_min_chunk - 1) / m->attn_min_chunk);
        p.merge_in_o = splits > 1 && (size_t)c.n_heads * splits * (c.head_dim + 2) * 8u <= 48u * 1024u ? 1 : 0;
    }
    p.merge_dist = 1;
    p.piece_pos = P.piece_pos;
    p.hd_shift = 0;
    while ((1 << p.hd_shift) < c.head_dim) ++p.hd_shift;
    p.lds_tasks = P.lds_tasks;
    p.lds_rope = P.lds_rope;
    p.lds_qkv = P.lds_qkv;
    p.lds_bias = P.lds_bias;
    p.lds_xs = P.lds_xs;
    p.lds_xres = P.lds_xres;
    p.lds_attn = P.lds_attn;
    p.lds_ring = P.lds_ring;
    p.ring_bytes = P.ring_bytes;
    p.in_bytes = P.in_bytes;
    p.in_double = P.in_double;
    p.attn_hpi = P.attn_hpi;
    p.wfmt = m->weight_fmt;
    p.max_tasks = P.max_tasks;
    p.eps = c.rms_eps;
    p.scale = 1.0f / std::sqrt((float)c.head_dim);
    p.inv_h = 1.0f / (float)c.hidden;
    p.token = token;
    p.pos = pos;
    p.tag0 = m->seq * (uint32_t)P.iv.size() + 1u;
    p.step_from_ws = 0;
    p.barrier = m->sync_mode == MBK_SYNC_BARRIER;
    p.epoch_base = m->epoch;
    p.spin_limit = m->spin_limit;
    p.skip_wg = m->skip_wg;
    p.skip_interval = m->skip_interval;
    p.first_iv = 0;
    p.last_iv = p.n_intervals;
    return p;
}

int check_step_args(const mbk_model *m, int32_t token, int32_t pos, const int32_t *argmax) {
    if (!m) return fail(MBK_ERR_ARG, "null model");
    if (!m->blob || !m->kv || !m->ws) return fail(MBK_ERR_STATE, "weights not packed or KV/workspace not bound");
    if (!argmax) return fail(MBK_ERR_ARG, "argmax output is null");
    if (token != MBK_TOKEN_PREV && (token < 0 || token >= m->c.vocab))
        return fail(MBK_ERR_ARG, "token %d outside [0, %d)", token, m->c.vocab);
    if (pos < 0 || pos >= m->c.kv_capacity) return fail(MBK_ERR_RANGE, "pos %d outside [0, %d)", pos, m->c.kv_capacity);
    return MBK_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// One launch of the persistent kernel for p, as the handle's launch mode says.
int launch_persistent(const mbk_model *m, Params &p, void *stream) {
    if (m->launch_mode == MBK_LAUNCH_COOPERATIVE) {
        void *args[] = {&p};
        HIPCHK(hipLaunchCooperativeKernel((const void *)kPersistent[p.gqa - 1], dim3(m->n_wg), dim3(kThreads), args,
                                          (unsigned)m->plan.lds_bytes, (hipStream_t)stream));
    } else {
        hipLaunchKernelGGL(kPersistent[p.gqa - 1], dim3(m->n_wg), dim3(kThreads), (unsigned)m->plan.lds_bytes,
                           (hipStream_t)stream, p);
        HIPCHK(hipGetLastError());
    }
    return MBK_OK;
}

int pack_matrix(mbk_model *m, const MatGeom &g, const void *s0, const void *s1, const void *s2, hipStream_t st) {
    const int hd = m->c.head_dim, nq_rows = m->c.n_heads * hd, nkv_rows = m->c.n_kv_heads * hd;
    const uint64_t n = (uint64_t)g.ntiles * g.IT * 64u;
    const int threads = 256;
    const int blocks = (int)std::min<uint64_t>((n + threads - 1) / threads, 65536);
    const uint16_t *a = (const uint16_t *)s0, *b = (const uint16_t *)s1, *d = (const uint16_t *)s2;
    if (g.fmt == FMT_FP8) {
        const uint64_t ns = (uint64_t)g.ntiles * ((g.tb - g.IT * 1024) / 4);
        const int bs = (int)std::min<uint64_t>((ns + threads - 1) / threads, 65536);
        hipLaunchKernelGGL(k_pack_scale, dim3(bs), dim3(threads), 0, st, m->blob, g, a, b, d, hd, nq_rows, nkv_rows);
        hipLaunchKernelGGL(k_pack_fp8, dim3(blocks), dim3(threads), 0, st, m->blob, g, a, b, d, hd, nq_rows, nkv_rows);
    } else {
        hipLaunchKernelGGL(k_pack, dim3(blocks), dim3(threads), 0, st, m->blob, g, a, b, d, hd, nq_rows, nkv_rows);
    }
    HIPCHK(hipGetLastError());
    return MBK_OK;
}

void drop_graph(mbk_model *m) {
    if (m->gexec) (void)hipGraphExecDestroy(m->gexec);
    if (m->graph) (void)hipGraphDestroy(m->graph);
    m->gexec = nullptr;
    m->graph = nullptr;
    m->node0 = nullptr;
}

}  // namespace

extern "C" {

const char *mbk_last_error(void) { return g_err.c_str(); }

int mbk_create(const mbk_config *cfg, mbk_model **out) {
    if (!cfg || !out) return fail(MBK_ERR_ARG, "null argument");
    const mbk_config &c = *cfg;
    if (c.n_layers <= 0 || c.hidden <= 0 || c.n_heads <= 0 || c.n_kv_heads <= 0 || c.head_dim <= 0 ||
        c.intermediate <= 0 || c.vocab <= 0 || c.kv_capacity <= 0)
        return fail(MBK_ERR_ARG, "every dimension must be positive");
    if (!(c.rms_eps > 0.f) || !(c.rope_theta > 0.f)) return fail(MBK_ERR_ARG, "rms_eps and rope_theta must be > 0");
    if (c.qkv_bias != 0 && c.qkv_bias != 1) return fail(MBK_ERR_ARG, "qkv_bias must be 0 or 1");
    if (c.head_dim != 16 && c.head_dim != 32 && c.head_dim != 64 && c.head_dim != 128)
        return fail(MBK_ERR_UNSUPPORTED, "head_dim %d not in {16, 32, 64, 128}", c.head_dim);
    if (c.n_heads % c.n_kv_heads != 0) return fail(MBK_ERR_UNSUPPORTED, "n_heads %% n_kv_heads != 0");
    if (c.n_heads / c.n_kv_heads > kMaxGqa) return fail(MBK_ERR_UNSUPPORTED, "more than %d query heads per KV head", kMaxGqa);
    if (c.n_kv_heads > 255) return fail(MBK_ERR_UNSUPPORTED, "more than 255 KV heads");
    const int Q = c.n_heads * c.head_dim;
    if (c.hidden % 8 || Q % 8 || c.intermediate % 8) return fail(MBK_ERR_UNSUPPORTED, "hidden, heads*head_dim and intermediate must be multiples of 8");
    if (c.hidden > kMaxVec || Q > kMaxVec || c.intermediate > kMaxVec)
        return fail(MBK_ERR_UNSUPPORTED, "vectors longer than %d", kMaxVec);
    if (c.kv_capacity > 8192) return fail(MBK_ERR_UNSUPPORTED, "kv_capacity %d > 8192", c.kv_capacity);
    if ((int64_t)c.vocab * c.hidden > ((int64_t)1 << 33)) return fail(MBK_ERR_UNSUPPORTED, "embedding too large");
    mbk_model *m = new mbk_model();
    m->c = c;
    *out = m;
    return MBK_OK;
}

void mbk_destroy(mbk_model *m) {
    if (!m) return;
    drop_graph(m);
    delete m;
}

int mbk_num_intervals(const mbk_model *m, int32_t *n) {
    if (!m || !n) return fail(MBK_ERR_ARG, "null argument");
    *n = 5 * m->c.n_layers + 1;
    return MBK_OK;
}

int mbk_set_debug(mbk_model *m, int32_t spin_limit, int32_t skip_wg, int32_t skip_interval) {
    if (!m || spin_limit < 0) return fail(MBK_ERR_ARG, "bad debug arguments");
    m->spin_limit = spin_limit ? spin_limit : (1 << 22);
    m->skip_wg = skip_wg;
    m->skip_interval = skip_interval;
    return MBK_OK;
}

int mbk_pack_weights(mbk_model *m, const mbk_weights *src, void *dst, size_t *dst_bytes, void *stream) {
    if (!m || !dst_bytes) return fail(MBK_ERR_ARG, "null argument");
    int rc = ensure_plan(m);
    if (rc) return rc;
    const Plan &P = m->plan;
    if (!dst) {
        *dst_bytes = P.total;
        return MBK_OK;
    }
    if (!src) return fail(MBK_ERR_ARG, "null weights");
    if (*dst_bytes < P.total) return fail(MBK_ERR_SIZE, "packed buffer %zu < %llu bytes", *dst_bytes, (unsigned long long)P.total);
    if (!aligned(dst, 256)) return fail(MBK_ERR_ARG, "packed buffer not 256-byte aligned");
    const mbk_config &c = m->c;
    auto ok16 = [](const void *p) { return p && aligned(p, 16); };
    if (!ok16(src->embed) || !ok16(src->final_norm)) return fail(MBK_ERR_ARG, "embed/final_norm null or misaligned");
    if (!src->attn_norm || !src->wq || !src->wk || !src->wv || !src->wo || !src->mlp_norm || !src->wgate ||
        !src->wup || !src->wdown || (c.qkv_bias && (!src->bq || !src->bk || !src->bv)))
        return fail(MBK_ERR_ARG, "null per-layer weight array");
    for (int l = 0; l < c.n_layers; ++l) {
        const void *ps[] = {src->attn_norm[l], src->wq[l], src->wk[l], src->wv[l], src->wo[l], src->mlp_norm[l],
                            src->wgate[l], src->wup[l], src->wdown[l]};
        for (const void *p : ps)
            if (!ok16(p)) return fail(MBK_ERR_ARG, "layer %d: weight pointer null or not 16-byte aligned", l);
        if (c.qkv_bias && (!src->bq[l] || !src->bk[l] || !src->bv[l])) return fail(MBK_ERR_ARG, "layer %d: null bias", l);
    }
    hipStream_t st = (hipStream_t)stream;
    drop_graph(m);
    m->blob = (uint8_t *)dst;
    const int hd = c.head_dim, Q = c.n_heads * hd, KV = c.n_kv_heads * hd;
    for (int l = 0; l < c.n_layers; ++l) {
        const LayerPlan &L = P.layers[l];
        if ((rc = pack_matrix(m, L.qkv, src->wq[l], src->wk[l], src->wv[l], st))) return rc;
        if ((rc = pack_matrix(m, L.o, src->wo[l], nullptr, nullptr, st))) return rc;
        if ((rc = pack_matrix(m, L.gu, src->wgate[l], src->wup[l], nullptr, st))) return rc;
        if ((rc = pack_matrix(m, L.down, src->wdown[l], nullptr, nullptr, st))) return rc;
        HIPCHK(hipMemcpyAsync(m->blob + L.attn_norm, src->attn_norm[l], 2u * c.hidden, hipMemcpyDeviceToDevice, st));
        HIPCHK(hipMemcpyAsync(m->blob + L.mlp_norm, src->mlp_norm[l], 2u * c.hidden, hipMemcpyDeviceToDevice, st));
        if (c.qkv_bias) {
            HIPCHK(hipMemcpyAsync(m->blob + L.bias, src->bq[l], 2u * Q, hipMemcpyDeviceToDevice, st));
            HIPCHK(hipMemcpyAsync(m->blob + L.bias + 2u * Q, src->bk[l], 2u * KV, hipMemcpyDeviceToDevice, st));
            HIPCHK(hipMemcpyAsync(m->blob + L.bias + 2u * (Q + KV), src->bv[l], 2u * KV, hipMemcpyDeviceToDevice, st));
        }
    }
    if ((rc = pack_matrix(m, P.embed, src->embed, nullptr, nullptr, st))) return rc;
    if (P.lmhead.off != P.embed.off && (rc = pack_matrix(m, P.lmhead, src->embed, nullptr, nullptr, st))) return rc;
    HIPCHK(hipMemcpyAsync(m->blob + P.final_norm, src->final_norm, 2u * c.hidden, hipMemcpyDeviceToDevice, st));
    HIPCHK(hipMemcpyAsync(m->blob + P.rope, m->rope_host.data(), m->rope_host.size() * 4, hipMemcpyHostToDevice, st));
    HIPCHK(hipMemcpyAsync(m->blob + P.table, P.iv.data(), P.iv.size() * sizeof(Interval), hipMemcpyHostToDevice, st));
    HIPCHK(hipMemcpyAsync(m->blob + P.tasks, P.task_list.data(), P.task_list.size() * sizeof(Task), hipMemcpyHostToDevice, st));
    HIPCHK(hipMemcpyAsync(m->blob + P.task_idx, P.task_index.data(), P.task_index.size() * sizeof(int32_t),
                          hipMemcpyHostToDevice, st));
    HIPCHK(hipStreamSynchronize(st));  // host-side sources above must outlive the copies
    return MBK_OK;
}

int mbk_alloc_kv(mbk_model *m, void *kv, size_t *kv_bytes, void *ws, size_t *ws_bytes, void *stream) {
    if (!m || !kv_bytes || !ws_bytes) return fail(MBK_ERR_ARG, "null argument");
    int rc = ensure_plan(m);
    if (rc) return rc;
    const mbk_config &c = m->c;
    const size_t need_kv = (size_t)c.n_layers * 2 * c.n_kv_heads * c.kv_capacity * c.head_dim * 2;
    const size_t need_ws = m->plan.ws.total;
    if (!kv || !ws) {
        *kv_bytes = need_kv;
        *ws_bytes = need_ws;
        return MBK_OK;
    }
    if (*kv_bytes < need_kv || *ws_bytes < need_ws)
        return fail(MBK_ERR_SIZE, "KV %zu < %zu or workspace %zu < %zu bytes", *kv_bytes, need_kv, *ws_bytes, need_ws);
    if (!aligned(kv, 256) || !aligned(ws, 256)) return fail(MBK_ERR_ARG, "KV/workspace not 256-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    HIPCHK(hipMemsetAsync(kv, 0, need_kv, st));
    HIPCHK(hipMemsetAsync(ws, 0, need_ws, st));
    drop_graph(m);
    m->kv = (uint16_t *)kv;
    m->ws = (uint8_t *)ws;
    m->epoch = 0;
    m->seq = 0;
    return MBK_OK;
}

int mbk_decode_step(mbk_model *m, int32_t token, int32_t pos, float *logits, int32_t *argmax, void *stream) {
    int rc = check_step_args(m, token, pos, argmax);
    if (rc || (rc = ensure_kernels(m))) return rc;
    next_seq(m);
    Params p = make_params(m, token, pos, logits, argmax);
    if ((rc = launch_persistent(m, p, stream))) return rc;
    if (p.barrier) m->epoch += (uint32_t)(p.n_intervals - 1);
    return MBK_OK;
}

int mbk_decode_step_static(mbk_model *m, void *kv, int32_t token, int32_t pos, float *logits, int32_t *argmax,
                           void *stream) {
    if (!m) return fail(MBK_ERR_ARG, "null model");
    int rc = ensure_plan(m);
    if (rc) return rc;
    if (m->plan.ws.total > kStaticScratchBytes)
        return fail(MBK_ERR_SIZE, "this shape needs a %llu-byte workspace; the static scratch holds %zu bytes "
                    "(use mbk_decode_step with a caller workspace)", (unsigned long long)m->plan.ws.total,
                    kStaticScratchBytes);
    if (!m->blob) return fail(MBK_ERR_STATE, "weights not packed");
    if (!kv || !aligned(kv, 256)) return fail(MBK_ERR_ARG, "KV cache null or not 256-byte aligned");
    if (!argmax) return fail(MBK_ERR_ARG, "argmax output is null");
    if (token != MBK_TOKEN_PREV && (token < 0 || token >= m->c.vocab))
        return fail(MBK_ERR_ARG, "token %d outside [0, %d)", token, m->c.vocab);
    if (pos < 0 || pos >= m->c.kv_capacity) return fail(MBK_ERR_RANGE, "pos %d outside [0, %d)", pos, m->c.kv_capacity);
    if ((rc = ensure_kernels(m))) return rc;
    int dev = 0;
    HIPCHK(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lock(g_static_mu);
    if ((int)g_static.size() <= dev) g_static.resize((size_t)dev + 1);
    StaticScratch &S = g_static[(size_t)dev];
    if (!S.ptr) {
        void *ptr = nullptr;
        HIPCHK(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
        S.ptr = (uint8_t *)ptr;
    }
    const uint32_t n_iv = (uint32_t)m->plan.iv.size();
    hipStream_t st = (hipStream_t)stream;
    if (!S.clean || S.next_tag > 0xffffffffu - 2u * n_iv) {
        // first use, an error seen by mbk_check, or tags about to wrap: start from a zeroed workspace
        hipLaunchKernelGGL(k_zero16, dim3(128), dim3(256), 0, st, S.ptr, (uint64_t)kStaticScratchBytes);
        HIPCHK(hipGetLastError());
        S.next_tag = 1;
        S.epoch = 0;
        S.clean = true;
    }
    Params p = make_params(m, token, pos, logits, argmax);
    p.kv = (uint16_t *)kv;
    p.ws = S.ptr;
    p.tag0 = S.next_tag;
    p.epoch_base = S.epoch;
    if ((rc = launch_persistent(m, p, stream))) return rc;
    S.next_tag += n_iv;
    if (p.barrier) S.epoch += n_iv - 1u;
    m->static_dev = dev;
    return MBK_OK;
}

int mbk_decode_step_ablation(mbk_model *m, int32_t token, int32_t pos, float *logits, int32_t *argmax,
                             int32_t use_graph, void *stream) {
    int rc = check_step_args(m, token, pos, argmax);
    if (rc || (rc = ensure_kernels(m))) return rc;
    hipStream_t st = (hipStream_t)stream;
    next_seq(m);
    Params p = make_params(m, token, pos, logits, argmax);
    p.barrier = 0;
    p.merge_dist = 0;  // a launch of one interval: its workgroups never wait for each other
    const unsigned lds = (unsigned)m->plan.lds_bytes;
    if (!use_graph) {
        for (int i = 0; i < p.n_intervals; ++i) {
            Params pi = p;
            pi.first_iv = i;
            pi.last_iv = i + 1;
            hipLaunchKernelGGL(kInterval[p.gqa - 1], dim3(m->n_wg), dim3(kThreads), lds, st, pi);
        }
        HIPCHK(hipGetLastError());
        return MBK_OK;
    }
    if (m->gexec && (m->g_logits != logits || m->g_argmax != argmax)) drop_graph(m);
    if (!m->gexec) {
        HIPCHK(hipGraphCreate(&m->graph, 0));
        hipGraphNode_t prev = nullptr;
        std::vector<Params> ps(p.n_intervals, p);
        for (int i = 0; i < p.n_intervals; ++i) {
            ps[i].step_from_ws = i == 0 ? 0 : 1;
            ps[i].first_iv = i;
            ps[i].last_iv = i + 1;
            void *kargs[] = {&ps[i]};
            hipKernelNodeParams kp{};
            kp.func = (void *)kInterval[p.gqa - 1];
            kp.gridDim = dim3(m->n_wg);
            kp.blockDim = dim3(kThreads);
            kp.sharedMemBytes = lds;
            kp.kernelParams = kargs;
            hipGraphNode_t node;
            HIPCHK(hipGraphAddKernelNode(&node, m->graph, prev ? &prev : nullptr, prev ? 1 : 0, &kp));
            if (i == 0) m->node0 = node;
            prev = node;
        }
        HIPCHK(hipGraphInstantiate(&m->gexec, m->graph, nullptr, nullptr, 0));
        m->g_logits = logits;
        m->g_argmax = argmax;
    }
    p.first_iv = 0;
    p.last_iv = 1;
    void *kargs[] = {&p};
    hipKernelNodeParams kp{};
    kp.func = (void *)kInterval[p.gqa - 1];
    kp.gridDim = dim3(m->n_wg);
    kp.blockDim = dim3(kThreads);
    kp.sharedMemBytes = lds;
    kp.kernelParams = kargs;
    HIPCHK(hipGraphExecKernelNodeSetParams(m->gexec, m->node0, &kp));
    HIPCHK(hipGraphLaunch(m->gexec, st));
    return MBK_OK;
}

int mbk_check(mbk_model *m, void *stream) {
    if (!m) return fail(MBK_ERR_ARG, "null model");
    HIPCHK(hipStreamSynchronize((hipStream_t)stream));
    if (m->static_dev >= 0) {
        // the static scratch this handle last stepped on (its error word is the first word)
        uint8_t *ptr = nullptr;
        {
            std::lock_guard<std::mutex> lock(g_static_mu);
            ptr = g_static[(size_t)m->static_dev].ptr;
        }
        uint32_t err = 0;
        HIPCHK(hipMemcpy(&err, ptr + m->plan.ws.ctrl, 4, hipMemcpyDeviceToHost));
        if (err) {
            std::lock_guard<std::mutex> lock(g_static_mu);
            g_static[(size_t)m->static_dev].clean = false;   // the next static step clears it first
            return fail(MBK_ERR_TIMEOUT, "a bounded device wait expired in a static-scratch step");
        }
    }
    if (!m->ws) return MBK_OK;
    uint32_t err = 0;
    HIPCHK(hipMemcpy(&err, m->ws + m->plan.ws.ctrl, 4, hipMemcpyDeviceToHost));
    if (err) return fail(MBK_ERR_TIMEOUT, "a bounded device wait expired; re-bind KV/workspace");
    return MBK_OK;
}

int mbk_set_phase_trace(mbk_model *m, void *buf, size_t bytes) {
    if (!m) return fail(MBK_ERR_ARG, "null model");
    if (!buf) {
        m->trace = nullptr;
        return MBK_OK;
    }
    int rc = ensure_plan(m);
    if (rc) return rc;
    const size_t need = m->plan.iv.size() * (size_t)m->n_wg * 4 * sizeof(uint64_t);
    if (bytes < need) return fail(MBK_ERR_SIZE, "phase trace buffer %zu < %zu bytes", bytes, need);
    if (!aligned(buf, 8)) return fail(MBK_ERR_ARG, "phase trace buffer not 8-byte aligned");
    drop_graph(m);
    m->trace = (uint64_t *)buf;
    return MBK_OK;
}

int mbk_set_sync_mode(mbk_model *m, int32_t mode) {
    if (!m) return fail(MBK_ERR_ARG, "null model");
    if (mode != MBK_SYNC_DATAFLOW && mode != MBK_SYNC_BARRIER) return fail(MBK_ERR_ARG, "unknown sync mode %d", mode);
    m->sync_mode = mode;
    return MBK_OK;
}

int mbk_set_launch_mode(mbk_model *m, int32_t mode) {
    if (!m) return fail(MBK_ERR_ARG, "null model");
    if (mode != MBK_LAUNCH_PLAIN && mode != MBK_LAUNCH_COOPERATIVE) return fail(MBK_ERR_ARG, "unknown launch mode %d", mode);
    m->launch_mode = mode;
    return MBK_OK;
}

int mbk_set_attention_split(mbk_model *m, int32_t min_positions) {
    if (!m || min_positions < 1) return fail(MBK_ERR_ARG, "min_positions must be >= 1");
    drop_graph(m);
    m->attn_min_chunk = min_positions;
    return MBK_OK;
}

int mbk_barrier_bench(mbk_model *m, int32_t n, void *stream, float *us_per_barrier) {
    if (!m || !us_per_barrier || n <= 0) return fail(MBK_ERR_ARG, "bad arguments");
    if (!m->ws || !m->blob) return fail(MBK_ERR_STATE, "workspace not bound");
    int rc = ensure_kernels(m);
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    hipEvent_t e0, e1;
    HIPCHK(hipEventCreate(&e0));
    HIPCHK(hipEventCreate(&e1));
    float t[2] = {0, 0};
    const int counts[2] = {0, n};
    for (int k = 0; k < 2; ++k) {
        Params p = make_params(m, 0, 0, nullptr, nullptr);
        int cnt = counts[k];
        void *args[] = {&p, &cnt};
        HIPCHK(hipEventRecord(e0, st));
        HIPCHK(hipLaunchCooperativeKernel((const void *)k_barrier_bench, dim3(m->n_wg), dim3(kThreads), args, 0, st));
        HIPCHK(hipEventRecord(e1, st));
        HIPCHK(hipEventSynchronize(e1));
        HIPCHK(hipEventElapsedTime(&t[k], e0, e1));
        m->epoch += (uint32_t)cnt;
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    *us_per_barrier = (t[1] - t[0]) * 1000.f / (float)n;
    return MBK_OK;
}

int mbk_get_matrix_layout(mbk_model *m, int32_t layer, int32_t which, mbk_matrix_layout *out) {
    if (!m || !out) return fail(MBK_ERR_ARG, "null argument");
    int rc = ensure_plan(m);
    if (rc) return rc;
    const Plan &P = m->plan;
    const MatGeom *g = nullptr;
    if (layer == -1 && which == 0) g = &P.embed;
    else if (layer == -1 && which == 1) g = &P.lmhead;
    else if (layer >= 0 && layer < m->c.n_layers && which >= 0 && which < 4) {
        const LayerPlan &L = P.layers[(size_t)layer];
        g = which == 0 ? &L.qkv : which == 1 ? &L.o : which == 2 ? &L.gu : &L.down;
    }
    if (!g) return fail(MBK_ERR_RANGE, "no matrix (layer %d, which %d)", layer, which);
    out->offset = g->off;
    out->rows = g->rows;
    out->cols = g->K;
    out->lanes_per_row = g->L;
    out->rows_per_tile = g->RT;
    out->steps = g->IT;
    out->tiles = g->ntiles;
    out->kind = g->kind;
    out->format = g->fmt;
    out->values_per_group = g->gv;
    out->tile_bytes = g->tb;
    out->scale_offset = g->fmt == FMT_FP8 ? g->IT * 1024 : -1;
    return MBK_OK;
}

}  // extern "C"

#include "prefill_host.h"

extern "C" {

int mbk_barrier_stress(mbk_model *m, int32_t n, void *stream, int32_t *first_bad) {
    if (!m || !first_bad || n <= 0) return fail(MBK_ERR_ARG, "bad arguments");
    if (!m->ws || !m->blob) return fail(MBK_ERR_STATE, "workspace not bound");
    int rc = ensure_kernels(m);
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *res = (uint32_t *)(m->ws + m->plan.ws.stress);
    const uint32_t init[4] = {0xffffffffu, 0u, 0u, 0u};
    HIPCHK(hipMemsetAsync(res + 4, 0, 4u * (size_t)m->n_wg, st));
    HIPCHK(hipMemcpyAsync(res, init, sizeof init, hipMemcpyHostToDevice, st));
    Params p = make_params(m, 0, 0, nullptr, nullptr);
    int cnt = n;
    uint32_t *slots = res + 4;
    void *args[] = {&p, &cnt, &res, &slots};
    HIPCHK(hipLaunchCooperativeKernel((const void *)k_barrier_stress, dim3(m->n_wg), dim3(kThreads), args, 0, st));
    m->epoch += (uint32_t)n;
    uint32_t out[4];
    HIPCHK(hipMemcpyAsync(out, res, sizeof out, hipMemcpyDeviceToHost, st));
    HIPCHK(hipStreamSynchronize(st));
    uint32_t err = 0;
    HIPCHK(hipMemcpy(&err, m->ws + m->plan.ws.ctrl, 4, hipMemcpyDeviceToHost));
    first_bad[0] = out[0] == 0xffffffffu ? 0 : (int32_t)out[0];
    first_bad[1] = (int32_t)out[1];
    first_bad[2] = (int32_t)out[2];
    first_bad[3] = (int32_t)out[3];
    if (err) return fail(MBK_ERR_TIMEOUT, "a grid barrier wait expired; re-bind KV/workspace");
    return MBK_OK;
}

int mbk_set_workgroups(mbk_model *m, int32_t n) {
    if (!m || n < 0) return fail(MBK_ERR_ARG, "bad arguments");
    if (m->planned && n != (m->n_wg_set ? m->n_wg_set : m->n_wg) && !(n == 0 && m->n_wg_set == 0))
        return fail(MBK_ERR_STATE, "the schedule is already planned for %d workgroups", m->n_wg);
    if (n > 0 && n < 1) return fail(MBK_ERR_ARG, "need at least one workgroup");
    m->n_wg_set = n;
    return MBK_OK;
}

int mbk_set_attention_items(mbk_model *m, int32_t heads_per_item) {
    if (!m) return fail(MBK_ERR_ARG, "bad arguments");
    const int G = m->c.n_heads / m->c.n_kv_heads;
    if (heads_per_item != 0 && heads_per_item != 1 && heads_per_item != G)
        return fail(MBK_ERR_ARG, "heads_per_item must be 0, 1 or %d (the query heads of a KV head)", G);
    if (m->planned && heads_per_item != m->attn_items_set)
        return fail(MBK_ERR_STATE, "the schedule is already planned");
    m->attn_items_set = heads_per_item;
    return MBK_OK;
}

int mbk_set_weight_format(mbk_model *m, int32_t format) {
    if (!m || (format != MBK_WEIGHTS_BF16 && format != MBK_WEIGHTS_FP8_E4M3))
        return fail(MBK_ERR_ARG, "format must be MBK_WEIGHTS_BF16 or MBK_WEIGHTS_FP8_E4M3");
    const int f = format == MBK_WEIGHTS_FP8_E4M3 ? FMT_FP8 : FMT_BF16;
    if (m->planned && f != m->weight_fmt) return fail(MBK_ERR_STATE, "the schedule is already planned");
    m->weight_fmt = f;
    return MBK_OK;
}

int mbk_describe(mbk_model *m, char *buf, size_t len) {
    if (!m || !buf || len == 0) return fail(MBK_ERR_ARG, "bad arguments");
    int rc = ensure_plan(m);
    if (rc) return rc;
    const Plan &P = m->plan;
    size_t tile_max = 0, task_max = 0;
    for (const Interval &v : P.iv)
        if (v.op != OP_ATTN) tile_max = std::max(tile_max, (size_t)v.mat.tb);
    for (const Task &t : P.task_list)
        if (P.iv[t.iv].op != OP_ATTN) task_max = std::max(task_max, (size_t)t.n * P.iv[t.iv].mat.tb);
    const int n = snprintf(buf, len,
        "{\"workgroups\": %d, \"threads\": %d, \"compute_waves\": %d, \"loader_waves\": %d, \"intervals\": %zu, "
        "\"packed_bytes\": %llu, \"workspace_bytes\": %llu, \"lds_bytes\": %zu, \"ring_bytes\": %d, "
        "\"max_tasks\": %d, \"tasks\": %zu, \"max_task_bytes\": %zu, \"max_tile_bytes\": %zu, "
        "\"max_splits\": %d, \"piece_positions\": %d, \"double_inputs\": %d, \"attention_heads_per_item\": %d, "
        "\"weight_format\": \"%s\"}",
        m->n_wg, kThreads, kCW, kLW, P.iv.size(), (unsigned long long)P.total, (unsigned long long)P.ws.total,
        P.lds_bytes, P.ring_bytes, P.max_tasks, P.task_list.size(), task_max, tile_max, P.max_splits, P.piece_pos, P.in_double,
        P.attn_hpi, m->weight_fmt == FMT_FP8 ? "fp8_e4m3" : "bf16");
    if (n < 0 || (size_t)n >= len) return fail(MBK_ERR_SIZE, "description needs %d bytes", n + 1);
    return MBK_OK;
}

}  // extern "C"
