/*
 * planner_driver.cpp -- host sanitizer run of libmbk's host side: shape validation, the planner (packed
 * layout, interval table, task lists, LDS layout), the size queries and the argument checks of every entry
 * point.  Built with the host pass of the library instrumented by -fsanitize=address,undefined (test
 * infrastructure: tests/test_sanitizers.py).  The workgroup count is fixed, so no call reaches a device.
 */
#include <cstdio>
#include <cstring>
#include <vector>

#include "mbk.h"

namespace {

int failures = 0;

void expect(bool ok, const char *what) {
    if (!ok) {
        std::printf("FAILED: %s (%s)\n", what, mbk_last_error());
        ++failures;
    }
}

void plan_shape(const mbk_config &c, bool fits_static) {
    mbk_model *m = nullptr;
    expect(mbk_create(&c, &m) == MBK_OK, "create");
    if (!m) return;
    expect(mbk_set_workgroups(m, 256) == MBK_OK, "set_workgroups");
    std::vector<char> buf(8192);
    expect(mbk_describe(m, buf.data(), buf.size()) == MBK_OK, "describe");
    expect(mbk_describe(m, buf.data(), 8) == MBK_ERR_SIZE, "describe into a short buffer");
    size_t packed = 0, kvb = 0, wsb = 0;
    expect(mbk_pack_weights(m, nullptr, nullptr, &packed, nullptr) == MBK_OK && packed > 0, "packed size");
    expect(mbk_alloc_kv(m, nullptr, &kvb, nullptr, &wsb, nullptr) == MBK_OK && kvb > 0 && wsb > 0, "kv size");
    for (int l = -1; l < c.n_layers; ++l)
        for (int which = 0; which < (l < 0 ? 1 : 4); ++which) {
            mbk_matrix_layout g;
            expect(mbk_get_matrix_layout(m, l, which, &g) == MBK_OK, "matrix layout");
            expect(g.offset + (uint64_t)g.tiles * g.steps * 1024u <= packed, "matrix inside the blob");
        }
    mbk_matrix_layout g;
    expect(mbk_get_matrix_layout(m, c.n_layers, 0, &g) == MBK_ERR_RANGE, "layout of a missing layer");
    int32_t am = 0, n = 0;
    expect(mbk_num_intervals(m, &n) == MBK_OK && n == 5 * c.n_layers + 1, "interval count");
    expect(mbk_decode_step(m, 0, 0, nullptr, &am, nullptr) == MBK_ERR_STATE, "step before packing");
    expect(mbk_decode_step_ablation(m, 0, 0, nullptr, &am, 1, nullptr) == MBK_ERR_STATE, "ablation before packing");
    expect(mbk_decode_step_static(m, nullptr, 0, 0, nullptr, &am, nullptr) ==
               (fits_static ? MBK_ERR_STATE : MBK_ERR_SIZE), "static step checks");
    int32_t bad[4];
    expect(mbk_barrier_stress(m, 10, nullptr, bad) == MBK_ERR_STATE, "stress before binding");
    expect(mbk_set_attention_split(m, 0) == MBK_ERR_ARG, "attention split of 0");
    expect(mbk_set_sync_mode(m, 7) == MBK_ERR_ARG, "unknown sync mode");
    expect(mbk_set_workgroups(m, 128) == MBK_ERR_STATE, "workgroups after planning");
    mbk_destroy(m);
}

}  // namespace

int main() {
    const mbk_config shapes[] = {
        {2, 64, 4, 2, 16, 176, 512, 32, 0, 1e-5f, 1e4f},
        {30, 576, 9, 3, 64, 1536, 49152, 128, 0, 1e-5f, 1e4f},
        {30, 576, 9, 3, 64, 1536, 49152, 4096, 0, 1e-5f, 1e4f},
        {24, 896, 14, 2, 64, 4864, 151936, 128, 1, 1e-6f, 1e6f},
        {24, 2048, 32, 32, 64, 8192, 49152, 4096, 0, 1e-5f, 1e4f},
        {1, 2048, 32, 32, 64, 8192, 262144, 128, 0, 1e-5f, 1e4f},
    };
    for (const mbk_config &c : shapes) plan_shape(c, true);
    plan_shape(mbk_config{1, 4096, 64, 64, 128, 8192, 1024, 4096, 0, 1e-5f, 1e4f}, false);
    // shapes the kernels do not handle are errors, not slower paths
    mbk_model *m = nullptr;
    mbk_config c = shapes[0];
    c.head_dim = 48;
    expect(mbk_create(&c, &m) == MBK_ERR_UNSUPPORTED, "head_dim 48");
    c = shapes[0];
    c.kv_capacity = 16384;
    expect(mbk_create(&c, &m) == MBK_ERR_UNSUPPORTED, "kv capacity 16384");
    c = shapes[0];
    c.n_layers = 0;
    expect(mbk_create(&c, &m) == MBK_ERR_ARG, "zero layers");
    expect(mbk_create(nullptr, &m) == MBK_ERR_ARG, "null config");
    mbk_destroy(nullptr);
    std::printf("planner driver: %s\n", failures ? "FAILED" : "ok");
    return failures ? 1 : 0;
}
