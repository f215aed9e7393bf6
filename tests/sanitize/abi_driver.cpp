/*
 * Calls the C ABI's argument checks and size queries without a GPU, for a
 * build whose host code carries AddressSanitizer and UndefinedBehavior-
 * Sanitizer (test infrastructure; tests/test_sanitizers_cpu.py builds and
 * runs it).  Every call here must be refused (or answered) before anything
 * reaches the GPU.
 */
#include <stdio.h>
#include <string.h>

#include "bastion.h"
#include "bastion_verify.h"

#define EXPECT(c)                                                   \
    do {                                                            \
        if (!(c)) {                                                 \
            fprintf(stderr, "line %d: %s failed\n", __LINE__, #c); \
            return 1;                                               \
        }                                                           \
    } while (0)

int main() {
    EXPECT(bastion_abi_version() == BASTION_ABI_VERSION);
    for (int s = -1; s < 6; ++s) EXPECT(strlen(bastion_status_string(s)) > 0);
    EXPECT(bastion_workspace_bytes(0, 1, 4, 100, 4, 8, BASTION_F32) == 0);
    EXPECT(bastion_workspace_bytes(64, 1, 16, 151936, 8, 64, BASTION_BF16) > 0);
    EXPECT(bastion_workspace_bytes(16384, 16, 32, 524288, 32, 1023, BASTION_F32) > 0);
    void *fake = reinterpret_cast<void *>(1 << 20);
    bastion_tree_out out;
    memset(&out, 0, sizeof out);
    EXPECT(bastion_build_trees(nullptr, 1, 2, 4, 100, 100, 4, 8, 1, nullptr, 0, 1.0, nullptr, &out,
                               fake, 1 << 30, nullptr) == BASTION_EINVAL);
    EXPECT(bastion_build_trees(fake, 1, 2, 4, 100, 100, 4, 8, 1, nullptr, 0, 1.0, nullptr, &out,
                               fake, 1 << 30, nullptr) == BASTION_EINVAL);   // outputs missing
    EXPECT(bastion_build_trees(fake, 1, 2, 40, 100, 100, 4, 8, 1, nullptr, 0, 1.0, nullptr, nullptr,
                               fake, 1 << 30, nullptr) == BASTION_EINVAL);
    EXPECT(bastion_build_trees_noalloc(fake, 7, 2, 4, 100, 100, 4, 8, 1, nullptr, 0, 1.0, nullptr,
                                       &out, nullptr) == BASTION_EINVAL);
    EXPECT(bastion_budget_select(nullptr, nullptr, 1, 8, 1, nullptr, 0, 1.0, nullptr, nullptr,
                                 nullptr) == BASTION_EINVAL);
    EXPECT(bastion_tree_mask(nullptr, nullptr, 1, 8, nullptr, nullptr, nullptr, nullptr) ==
           BASTION_EINVAL);
    EXPECT(bastion_accept(nullptr, nullptr, nullptr, 1, 4, 8, nullptr, nullptr, nullptr, nullptr,
                          nullptr) == BASTION_EINVAL);
    bastion_mixture_out mo;
    memset(&mo, 0, sizeof mo);
    EXPECT(bastion_mixture_score(fake, 1, reinterpret_cast<const float *>(fake), 2, 17, 4, 100, 100,
                                 4, 8, &mo, nullptr, fake, 1 << 30, nullptr) == BASTION_EINVAL);
    bastion_marginal_out mg;
    memset(&mg, 0, sizeof mg);
    EXPECT(bastion_mixture_marginal(fake, 1, reinterpret_cast<const float *>(fake), 2, 3, 4, 100,
                                    100, 4, 8, &mg, nullptr, fake, 1 << 30, nullptr) ==
           BASTION_EINVAL);
    EXPECT(bastion_sample_nodes(nullptr, 1, 1, 8, 100, 100, nullptr, 1.0f, 0u, nullptr, nullptr) ==
           BASTION_EINVAL);
    EXPECT(bastion_sample_nodes(fake, 1, 1, 8, 100, 100, reinterpret_cast<const int32_t *>(fake),
                                -1.0f, 0u, reinterpret_cast<int32_t *>(fake), nullptr) ==
           BASTION_EINVAL);
    EXPECT(bastion_mixture_sample(nullptr, 1, 2, 1.0, nullptr, nullptr, 4, nullptr, nullptr,
                                  nullptr) == BASTION_EINVAL);
    EXPECT(bastion_tree_attention_workspace_bytes(1, 65, 32, 8, 9216) > 0);
    EXPECT(bastion_tree_attention_workspace_bytes(1, 65, 30, 8, 9216) == 0);
    EXPECT(bastion_tree_attention(nullptr, 0, 1, 65, 32, 8, 128, fake, fake, 9216, nullptr, -1,
                                  nullptr, nullptr, 3, nullptr, fake, fake, 1 << 30, nullptr) ==
           BASTION_EINVAL);
    bastion_set_tuning(3, 1);
    EXPECT(bastion_workspace_bytes(4, 1, 16, 4096, 8, 64, BASTION_BF16) > 0);
    bastion_set_tuning(0, -1);
    printf("abi driver ok\n");
    return 0;
}
