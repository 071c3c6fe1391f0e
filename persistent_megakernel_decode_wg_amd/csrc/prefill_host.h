// prefill_host.h -- host side of the multi-token prefill (scratch layout, GEMM dispatch, the launch sequence
// and its C entry points); included once by mbk.hip, after the model and plan types it uses.  The kernels are in
// prefill.h.
#pragma once

namespace {

// Scratch of a prefill of n tokens: token ids, residual stream, rotated queries, two hi/lo input buffers,
// the logits and the quarter sums of a k-split projection.  Rows are padded to whole position tiles.
struct PfLayout { size_t tok, x, q, in[4], logits, part, total; int Pp, ks; };

int round_up(int v, int m) { return (v + m - 1) / m * m; }

PfLayout pf_layout(const mbk_config &c, int n) {
    PfLayout L{};
    L.Pp = round_up(n, kPfTileP);
    const int Q = c.n_heads * c.head_dim;
    L.ks = std::max(round_up(c.hidden, 32), std::max(round_up(Q, 32), round_up(c.intermediate, 32)));
    size_t o = 0;
    L.tok = o; o = align256(o + 4u * (size_t)L.Pp);
    L.x = o; o = align256(o + 4u * (size_t)L.Pp * c.hidden);
    L.q = o; o = align256(o + 4u * (size_t)L.Pp * Q);
    for (int i = 0; i < 4; ++i) { L.in[i] = o; o = align256(o + 2u * (size_t)L.Pp * L.ks); }
    L.logits = o; o = align256(o + 4u * (size_t)c.vocab);
    L.part = o; o = align256(o + 16u * (size_t)L.Pp * std::max(c.hidden, Q + 2 * c.n_kv_heads * c.head_dim));
    L.total = o;
    return L;
}

constexpr unsigned kPfLMinGroups = 128;  // workgroups the shared-tile GEMM needs to fill the device
constexpr int kPfSplitMinK = 2048;       // inputs from which Q/K/V, output and down projections split their k steps
constexpr unsigned kPfSplitMinGroups = 64;  // 128-row tiles from which they do (x 4 workgroups)
constexpr size_t kPfOnePbWeights = (size_t)8 << 20;  // largest matrix whose per-wave GEMM takes one position block

// One shared-tile GEMM launch (its LDS above the default limit is allowed once per instance).
template <int OP, int WRB, bool SPLIT = false>
void pf_gemm_lds(const PfParams &pp, const MatGeom &g, int layer, int src, int dst, int np_rows, uint64_t bias,
                 hipStream_t st) {
    static bool lds_set = false;
    if (!lds_set) {
        (void)hipFuncSetAttribute((const void *)k_pf_gemm_lds<OP, WRB, SPLIT>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, PfLGeom<WRB>::kLds);
        lds_set = true;
    }
    const dim3 grid((unsigned)((g.rows + 32 * WRB - 1) / (32 * WRB)), (unsigned)(np_rows / 64), SPLIT ? 4u : 1u);
    hipLaunchKernelGGL((k_pf_gemm_lds<OP, WRB, SPLIT>), grid, dim3(256), (unsigned)PfLGeom<WRB>::kLds, st, pp, g,
                       layer, src, dst, np_rows, bias);
    if (SPLIT)
        hipLaunchKernelGGL(k_pf_split_sum<OP>, dim3((unsigned)((g.rows + 255) / 256), (unsigned)np_rows), dim3(256), 0,
                           st, pp, g, layer, dst, np_rows, bias);
}

// The per-wave kernel's launch shape (bf16 or fp8 weights alike): four row blocks and two position blocks per
// workgroup (every activation load feeds four products, every weight load two) while that leaves at least 256
// workgroups; else, for matrices of up to 8M weights, one position block per workgroup, and for larger ones
// two; with two row blocks while that leaves 256 workgroups, else one.
template <int OP, bool F8>
void pf_gemm_wave(const PfParams &pp, const MatGeom &g, int layer, int src, int dst, int np_rows, uint64_t bias,
                  hipStream_t st) {
    const unsigned py = (unsigned)((np_rows + kPfPos - 1) / kPfPos), p16 = (unsigned)(np_rows / 16);
    const unsigned x4 = (unsigned)((g.rows + 63) / 64), x2 = (unsigned)((g.rows + 31) / 32), x1 = (unsigned)((g.rows + 15) / 16);
    const bool one_pb = (size_t)g.rows * g.K <= kPfOnePbWeights;
    if (x4 * py >= 256)
        hipLaunchKernelGGL((k_pf_gemm<OP, 4, 4, F8, 2>), dim3(x4, py), dim3(256), 0, st, pp, g, layer, src, dst, np_rows, bias);
    else if (one_pb && x2 * p16 >= 256)
        hipLaunchKernelGGL((k_pf_gemm<OP, 2, 4, F8, 1>), dim3(x2, p16), dim3(256), 0, st, pp, g, layer, src, dst, np_rows, bias);
    else if (one_pb)
        hipLaunchKernelGGL((k_pf_gemm<OP, 1, 4, F8, 1>), dim3(x1, p16), dim3(256), 0, st, pp, g, layer, src, dst, np_rows, bias);
    else if (x2 * py >= 256)
        hipLaunchKernelGGL((k_pf_gemm<OP, 2, 4, F8, 2>), dim3(x2, py), dim3(256), 0, st, pp, g, layer, src, dst, np_rows, bias);
    else
        hipLaunchKernelGGL((k_pf_gemm<OP, 1, 4, F8, 2>), dim3(x1, py), dim3(256), 0, st, pp, g, layer, src, dst, np_rows, bias);
}

template <int OP>
void pf_gemm(const PfParams &pp, const MatGeom &g, int layer, int src, int dst, int np_rows, uint64_t bias, hipStream_t st) {
    // every matrix's k steps are split over four waves whatever the prompt length: the split fixes the order
    // in which a row's products are added, so a prompt's results do not depend on how it is cut into calls.
    // Long prompts over bf16 weights: operand tiles shared through LDS (128-row workgroup tiles, or 64-row ones
    // where the 128-row tiles would leave fewer than two workgroups per compute unit); else the per-wave kernel
    // (none of these choices changes the order; fp8 matrices always take the per-wave kernel, which widens
    // their codes)
    const unsigned pl = (unsigned)(np_rows / 64);
    const unsigned g4 = (unsigned)((g.rows + 127) / 128) * pl, g2 = (unsigned)((g.rows + 63) / 64) * pl;
    const bool lds_ok = g.fmt == FMT_BF16 && np_rows % 64 == 0;
    // query/key/value, output and down projections over wide inputs: the four k-step quarters on four workgroups each (four
    // times the workgroups, a quarter of the chain), their sums added in order by a second kernel
    constexpr bool kSplitOp = OP == OP_O || OP == OP_DOWN || OP == OP_QKV;
    if (kSplitOp && lds_ok && g.K >= kPfSplitMinK && g4 >= kPfSplitMinGroups && g4 < 512)
        pf_gemm_lds<OP, 4, kSplitOp>(pp, g, layer, src, dst, np_rows, bias, st);
    else if (lds_ok && g4 >= 512)
        pf_gemm_lds<OP, 4>(pp, g, layer, src, dst, np_rows, bias, st);
    else if (lds_ok && g2 >= 256 && g4 >= kPfLMinGroups)
        pf_gemm_lds<OP, 2>(pp, g, layer, src, dst, np_rows, bias, st);
    else if (lds_ok && g4 >= kPfLMinGroups)
        pf_gemm_lds<OP, 4>(pp, g, layer, src, dst, np_rows, bias, st);
    else if (g.fmt == FMT_FP8)
        pf_gemm_wave<OP, true>(pp, g, layer, src, dst, np_rows, bias, st);
    else
        pf_gemm_wave<OP, false>(pp, g, layer, src, dst, np_rows, bias, st);
}

}  // namespace

extern "C" {

int mbk_prefill_scratch_bytes(mbk_model *m, int32_t n_tokens, size_t *bytes) {
    if (!m || !bytes || n_tokens < 1) return fail(MBK_ERR_ARG, "bad arguments");
    if (n_tokens > m->c.kv_capacity) return fail(MBK_ERR_RANGE, "%d tokens exceed the %d-slot cache", n_tokens, m->c.kv_capacity);
    *bytes = pf_layout(m->c, n_tokens).total;
    return MBK_OK;
}

int mbk_prefill(mbk_model *m, const int32_t *tokens, int32_t n_tokens, int32_t pos0, void *scratch,
                size_t scratch_bytes, float *logits, int32_t *argmax, void *stream) {
    if (!m || !tokens || !argmax || n_tokens < 1) return fail(MBK_ERR_ARG, "bad arguments");
    const mbk_config &c = m->c;
    if (pos0 < 0 || (int64_t)pos0 + n_tokens > c.kv_capacity)
        return fail(MBK_ERR_RANGE, "positions %d..%d outside [0, %d)", pos0, pos0 + n_tokens - 1, c.kv_capacity);
    for (int i = 0; i < n_tokens; ++i)
        if (tokens[i] < 0 || tokens[i] >= c.vocab) return fail(MBK_ERR_ARG, "token %d at %d outside [0, %d)", tokens[i], i, c.vocab);
    if (!m->blob || !m->kv) return fail(MBK_ERR_STATE, "weights not packed or KV cache not bound");
    const PfLayout L = pf_layout(c, n_tokens);
    if (!scratch || scratch_bytes < L.total) return fail(MBK_ERR_SIZE, "prefill scratch %zu < %zu bytes", scratch_bytes, L.total);
    if (!aligned(scratch, 256)) return fail(MBK_ERR_ARG, "prefill scratch not 256-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    const Plan &P = m->plan;
    uint8_t *sc = (uint8_t *)scratch;
    HIPCHK(hipMemcpyAsync(sc + L.tok, tokens, 4u * (size_t)n_tokens, hipMemcpyHostToDevice, st));
    PfParams pp{};
    pp.blob = m->blob;
    pp.kv = m->kv;
    pp.tok = (const int32_t *)(sc + L.tok);
    pp.x = (float *)(sc + L.x);
    pp.q = (float *)(sc + L.q);
    pp.inh[0] = (uint16_t *)(sc + L.in[0]);
    pp.inl[0] = (uint16_t *)(sc + L.in[1]);
    pp.inh[1] = (uint16_t *)(sc + L.in[2]);
    pp.inl[1] = (uint16_t *)(sc + L.in[3]);
    pp.part = (float *)(sc + L.part);
    pp.logits = logits ? logits : (float *)(sc + L.logits);
    pp.argmax_out = argmax;
    pp.prev_token = m->ws ? (uint32_t *)(m->ws + P.ws.ctrl) + 1 : nullptr;
    pp.embed = P.embed;
    pp.rope = P.rope;
    pp.P = n_tokens;
    pp.Pp = L.Pp;
    pp.ks = L.ks;
    pp.pos0 = pos0;
    pp.H = c.hidden;
    pp.nq = c.n_heads;
    pp.nkv = c.n_kv_heads;
    pp.hd = c.head_dim;
    pp.I = c.intermediate;
    pp.V = c.vocab;
    pp.S = c.kv_capacity;
    pp.gqa = c.n_heads / c.n_kv_heads;
    pp.hd_shift = 0;
    while ((1 << pp.hd_shift) < c.head_dim) ++pp.hd_shift;
    pp.eps = c.rms_eps;
    pp.scale = 1.0f / std::sqrt((float)c.head_dim);
    const uint64_t none = ~(uint64_t)0;
    const int Q = c.n_heads * c.head_dim;
    for (int l = 0; l < c.n_layers; ++l) {
        const LayerPlan &Y = P.layers[(size_t)l];
        hipLaunchKernelGGL(k_pf_norm, dim3((unsigned)L.Pp), dim3(256), 0, st, pp, Y.attn_norm, 0, l == 0 ? 1 : 0, 0);
        pf_gemm<OP_QKV>(pp, Y.qkv, l, 0, 0, L.Pp, Y.bias, st);
        if (c.head_dim == 64 || c.head_dim == 128) {
            const dim3 grid((unsigned)((n_tokens + 15) / 16), (unsigned)c.n_heads);
            if (c.head_dim == 64) hipLaunchKernelGGL((k_pf_attn_mma<64, 4>), grid, dim3(256), 0, st, pp, l, 1);
            else hipLaunchKernelGGL((k_pf_attn_mma<128, 4>), grid, dim3(256), 0, st, pp, l, 1);
        } else {
            hipLaunchKernelGGL(k_pf_attn, dim3((unsigned)((n_tokens + kPfAttnQ - 1) / kPfAttnQ), (unsigned)c.n_heads),
                               dim3(256), 0, st, pp, l, 1);
        }
        if (Q % 32) hipLaunchKernelGGL(k_pf_clear_tail, dim3((unsigned)L.Pp), dim3(256), 0, st, pp, 1, Q);
        pf_gemm<OP_O>(pp, Y.o, l, 1, 0, L.Pp, none, st);
        hipLaunchKernelGGL(k_pf_norm, dim3((unsigned)L.Pp), dim3(256), 0, st, pp, Y.mlp_norm, 0, 0, 0);
        pf_gemm<OP_GATEUP>(pp, Y.gu, l, 0, 1, L.Pp, none, st);
        if (c.intermediate % 32) hipLaunchKernelGGL(k_pf_clear_tail, dim3((unsigned)L.Pp), dim3(256), 0, st, pp, 1, c.intermediate);
        pf_gemm<OP_DOWN>(pp, Y.down, l, 1, 0, L.Pp, none, st);
    }
    // the last position: final norm, tied vocabulary projection, argmax
    hipLaunchKernelGGL(k_pf_norm, dim3(1), dim3(256), 0, st, pp, P.final_norm, 0, 0, 1);
    pf_gemm<OP_LMHEAD>(pp, P.lmhead, -1, 0, 0, 16, none, st);
    hipLaunchKernelGGL(k_pf_argmax, dim3(1), dim3(1024), 0, st, pp);
    HIPCHK(hipGetLastError());
    return MBK_OK;
}

}  // extern "C"
