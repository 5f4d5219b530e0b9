// Host-side checks of the C ABI under AddressSanitizer and UndefinedBehavior-
// Sanitizer (built by tests/test_host_sanitizers.py from the library's
// sources compiled for the host only; no GPU is touched). Every call here
// either only plans (sizes, paths) or carries an argument the library must
// reject before any launch. Exit status 0 means every expectation held.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "qsa.h"

static int failures = 0;

static void expect(bool ok, const char *what, long long a = 0, long long b = 0)
{
    if (!ok) {
        std::fprintf(stderr, "FAILED: %s (%lld, %lld)\n", what, a, b);
        ++failures;
    }
}

int main()
{
    alignas(16) static float buf[64];
    alignas(16) static int32_t ibuf[64];
    alignas(16) static unsigned char ws[4096];
    float *fp = buf;
    int32_t *ip = ibuf;

    // Plans and workspace sizes over the argument space, including values
    // far past anything valid: no call may overflow or read out of bounds.
    const int32_t nqs[] = {-1, 0, 1, 3, 16, 17, 256, 65535, 65536, 0x7fffffff};
    const int32_t nbs[] = {-5, 0, 1, 63, 64, 4104, 4105, 65536, 1048576, 1048577, 1 << 29, 0x7fffffff};
    const int32_t bss[] = {-1, 0, 1, 3, 4, 7, 1 << 20, 0x7fffffff};
    const int32_t widths[] = {-1, 0, 1, 256, 2048, 16380, 16384, 1 << 30, 0x7fffffff};
    const int calls[] = {QSA_DECODE, QSA_PROMPT, 7};
    qsa_options opts[8];
    std::memset(opts, 0, sizeof opts);
    opts[1].topk_path = QSA_PATH_SPLIT;
    opts[1].chunk_blocks = 64;
    opts[2].topk_path = QSA_PATH_ONEREAD;
    opts[2].force_fallback = 1;
    opts[3].topk_path = QSA_PATH_FILTER;
    opts[3].filter_blocks = 1024;
    opts[4].topk_path = 99;                 // invalid path
    opts[5].chunk_blocks = 63;              // not a multiple of 4
    opts[6].sample = 7;                     // invalid sample mode
    opts[7].reserved[1] = 1;                // reserved must be zero
    long long planned = 0, rejected = 0;
    for (int32_t nq : nqs)
        for (int32_t nb : nbs)
            for (int32_t bs : bss)
                for (int32_t w : widths)
                    for (int c : calls)
                        for (int o = -1; o < 8; ++o) {
                            const qsa_options *op = o < 0 ? nullptr : &opts[o];
                            qsa_topk_plan p;
                            std::memset(&p, 0xAB, sizeof p);
                            const qsa_status s = qsa_topk_plan_get(nq, nb, bs, w, (qsa_call)c, op, &p);
                            const size_t bytes = qsa_topk_workspace_bytes(nq, nb, bs, w, (qsa_call)c, op);
                            if (s == QSA_OK) {
                                ++planned;
                                expect(p.path == QSA_PATH_SPLIT || p.path == QSA_PATH_ONEREAD ||
                                           p.path == QSA_PATH_FILTER, "plan path", nb, w);
                                expect(bytes == p.workspace_bytes, "workspace bytes match the plan", nb, w);
                                expect(p.r_blocks >= 0, "r_blocks", nb, w);
                                if (p.path == QSA_PATH_ONEREAD)
                                    expect(2 * ((long long)p.r_blocks + 1) <= p.cap, "one-read r bound", p.r_blocks);
                            } else {
                                ++rejected;
                                expect(bytes == 0, "rejected sizes give 0 bytes", nb, w);
                            }
                        }
    expect(qsa_topk_plan_get(3, 1000, 4, 256, QSA_DECODE, nullptr, nullptr) != QSA_OK, "plan without output");

    // Attention workspace sizes.
    const int32_t heads[] = {-1, 0, 1, 8, 16, 17, 64, 65536};
    for (int32_t nq : nqs)
        for (int32_t h : heads)
            for (int32_t kv : heads)
                for (int32_t w : widths) {
                    (void)qsa_selection_attention_workspace_bytes(nq, h, kv, w);
                    (void)qsa_selection_attention_shared_workspace_bytes(nq, h, kv, w);
                }

    // Arguments every entry point must reject before any launch.
    expect(qsa_block_topk(nullptr, 16, 1, 16, 4, 64, QSA_DECODE, nullptr, ip, ip, ws, sizeof ws, nullptr, nullptr) != QSA_OK,
           "topk: null scores");
    expect(qsa_block_topk(fp, 8, 1, 16, 4, 64, QSA_DECODE, nullptr, ip, ip, ws, sizeof ws, nullptr, nullptr) != QSA_OK,
           "topk: ld below n_blocks");
    expect(qsa_block_topk(fp, 16, 1, 16, 4, 64, QSA_DECODE, ip, ip, ip, ws, sizeof ws, nullptr, nullptr) != QSA_OK,
           "topk: active count on a decode call");
    expect(qsa_block_topk(fp, 16, 1, 16, 0, 64, QSA_DECODE, nullptr, ip, ip, ws, sizeof ws, nullptr, nullptr) != QSA_OK,
           "topk: block size 0");
    expect(qsa_topk_workspace_bytes(2, 1 << 20, 4, 2048, QSA_PROMPT, nullptr) > 16, "a filtered split needs workspace");
    expect(qsa_block_topk(fp, 1 << 20, 2, 1 << 20, 4, 2048, QSA_PROMPT, nullptr, ip, ip, ws, 16, nullptr, nullptr) ==
               QSA_EWORKSPACE, "topk: workspace too small");
    expect(qsa_block_topk(fp, 16, 1, 16, 4, 64, (qsa_call)5, nullptr, ip, ip, ws, sizeof ws, nullptr, nullptr) != QSA_OK,
           "topk: bad call");
    expect(qsa_block_topk_cells(fp, 16, 1, 16, 4, 64, QSA_DECODE, nullptr, ip, ip, ws, sizeof ws, nullptr, nullptr) !=
               QSA_OK, "topk cells: null lengths");
    expect(qsa_block_topk_noalloc(fp, 1 << 30, 256, 1 << 29, 1, 1 << 30, QSA_PROMPT, nullptr, ip, ip, nullptr) !=
               QSA_OK, "noalloc: past its array");
    expect(qsa_block_scores(fp, fp, fp, fp, 16, 1, 1, 64, 16, nullptr) != QSA_OK, "scores: head_dim 64");
    expect(qsa_block_scores(fp, fp, fp, fp, 8, 1, 1, 128, 16, nullptr) != QSA_OK, "scores: ld below n_blocks");
    expect(qsa_block_scores(nullptr, fp, fp, fp, 16, 1, 1, 128, 16, nullptr) != QSA_OK, "scores: null q");
    expect(qsa_block_scores_bf16(fp, fp, fp, fp, (int64_t)1 << 24, 2, 1, 128, 16, nullptr) != QSA_OK,
           "bf16 scores: ld of 2^24");
    expect(qsa_select(fp, fp, fp, 1, 128, fp, 16, 1, 16, 4, 64, QSA_DECODE, ip, ip, ip, ws, sizeof ws, nullptr,
                      nullptr) != QSA_OK, "select: active count on a decode call");
    expect(qsa_select_cells(fp, fp, fp, 1, 128, fp, 16, 1, 16, 4, 64, QSA_PROMPT, nullptr, ip, ip, ws, sizeof ws,
                            nullptr, nullptr) != QSA_OK, "select cells: null lengths");
    expect(qsa_selection_attention(fp, fp, fp, ip, 64, fp, fp, 2, 16, 3, 128, 256, 64, 0.1f, ws, sizeof ws,
                                   nullptr) != QSA_OK, "attention: heads not a multiple of kv heads");
    expect(qsa_selection_attention(fp, fp, fp, ip, 32, fp, fp, 2, 16, 2, 128, 256, 64, 0.1f, ws, sizeof ws,
                                   nullptr) != QSA_OK, "attention: ld_ids below width");
    expect(qsa_selection_attention_shared(fp, fp, fp, ip, 64, fp, fp, 2, 32, 2, 128, 256, 64, 0.1f, ws, sizeof ws,
                                          nullptr) != QSA_OK, "shared attention: groups of 16 heads");
    expect(qsa_selection_attention_shared(fp, fp, fp, ip, 8192, fp, fp, 2, 16, 2, 128, 1 << 20, 8192, 0.1f, ws,
                                          sizeof ws, nullptr) != QSA_OK, "shared attention: width past 4,096");

    for (int c = -1; c < 10; ++c)
        expect(qsa_status_str((qsa_status)c) != nullptr, "status string", c);

    std::printf("planned %lld, rejected %lld, failures %d\n", planned, rejected, failures);
    return failures == 0 ? 0 : 1;
}
