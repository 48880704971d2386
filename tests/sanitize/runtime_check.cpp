// runtime_check.cpp -- drives the host-side argument checks of the C ABI
// (include/lora_mi355x.h) under AddressSanitizer and UndefinedBehaviorSanitizer,
// with no GPU: every call below must return its documented status before the
// library touches a device.  Built (host code sanitized, device code as usual)
// and run by tests/test_sanitizers.py; not part of the library.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "lora_mi355x.h"

static int failures = 0;

static void expect(int got, int want, const char *what)
{
    if (got != want) {
        std::printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, lora_last_error(nullptr));
        ++failures;
    } else {
        std::printf("ok   %s: %s\n", what, lora_status_string(got));
    }
}

int main()
{
    lora_module_shape ok_shape[2] = {{4096, 4096}, {5120, 1024}};
    lora_module_shape bad_shape[1] = {{100, 4096}};
    lora_ctx *ctx = reinterpret_cast<lora_ctx *>(0x1);
    expect(lora_slots_create(nullptr, 8, 16, ok_shape, 2, LORA_BF16, 256, 0),
           LORA_ERR_INVALID_ARGUMENT, "create: out is NULL");
    expect(lora_slots_create(&ctx, 0, 16, ok_shape, 2, LORA_BF16, 256, 0),
           LORA_ERR_INVALID_ARGUMENT, "create: max_loras 0");
    if (ctx != nullptr) {
        std::printf("FAIL create: *out not cleared on error\n");
        ++failures;
    }
    expect(lora_slots_create(&ctx, LORA_MAX_SLOTS + 1, 16, ok_shape, 2, LORA_BF16, 256, 0),
           LORA_ERR_INVALID_ARGUMENT, "create: max_loras above the limit");
    expect(lora_slots_create(&ctx, 8, 0, ok_shape, 2, LORA_BF16, 256, 0),
           LORA_ERR_INVALID_ARGUMENT, "create: max_rank 0");
    expect(lora_slots_create(&ctx, 8, LORA_MAX_RANK + 1, ok_shape, 2, LORA_BF16, 256, 0),
           LORA_ERR_RANK_EXCEEDS_MAX, "create: max_rank above the limit");
    expect(lora_slots_create(&ctx, 8, 16, nullptr, 2, LORA_BF16, 256, 0),
           LORA_ERR_INVALID_ARGUMENT, "create: modules NULL");
    expect(lora_slots_create(&ctx, 8, 16, ok_shape, 0, LORA_BF16, 256, 0),
           LORA_ERR_INVALID_ARGUMENT, "create: no modules");
    expect(lora_slots_create(&ctx, 8, 16, ok_shape, 2, 7, 256, 0),
           LORA_ERR_INVALID_ARGUMENT, "create: unknown dtype");
    expect(lora_slots_create(&ctx, 8, 16, ok_shape, 2, LORA_BF16, 0, 0),
           LORA_ERR_INVALID_ARGUMENT, "create: max_tokens 0");
    expect(lora_slots_create(&ctx, 8, 16, bad_shape, 1, LORA_BF16, 256, 0),
           LORA_ERR_INVALID_ARGUMENT, "create: d_in not a multiple of 8");
    if (std::strstr(lora_last_error(nullptr), "multiples of 8") == nullptr) {
        std::printf("FAIL create: detail message '%s'\n", lora_last_error(nullptr));
        ++failures;
    }
    // every call taking a ctx rejects NULL
    const void *null_w[2] = {nullptr, nullptr};
    int32_t mods[1] = {0};
    const void *xs[1] = {nullptr};
    void *ys[1] = {nullptr};
    int32_t used[1] = {0};
    uint32_t flags = 0;
    lora_stats st;
    lora_profile pr;
    expect(lora_slot_load(nullptr, 0, null_w, null_w, 8, 16.0, 0), LORA_ERR_INVALID_ARGUMENT, "load: ctx NULL");
    expect(lora_slot_load_ex(nullptr, 0, null_w, null_w, nullptr, nullptr, 8, 16.0, 0),
           LORA_ERR_INVALID_ARGUMENT, "load_ex: ctx NULL");
    expect(lora_slot_load_saved(nullptr, 0, 0, null_w, nullptr), LORA_ERR_INVALID_ARGUMENT,
           "load_saved: ctx NULL");
    expect(lora_slot_clear(nullptr, 0), LORA_ERR_INVALID_ARGUMENT, "clear: ctx NULL");
    expect(lora_sync_loads(nullptr), LORA_ERR_INVALID_ARGUMENT, "sync_loads: ctx NULL");
    expect(lora_plan_prepare(nullptr, nullptr, 0, nullptr), LORA_ERR_INVALID_ARGUMENT, "plan: ctx NULL");
    expect(lora_plan_prepare_slots(nullptr, nullptr, 0, used, 1, nullptr), LORA_ERR_INVALID_ARGUMENT,
           "plan_slots: ctx NULL");
    expect(lora_shrink(nullptr, nullptr, 0, nullptr), LORA_ERR_INVALID_ARGUMENT, "shrink: ctx NULL");
    expect(lora_expand(nullptr, nullptr, 0, nullptr), LORA_ERR_INVALID_ARGUMENT, "expand: ctx NULL");
    expect(lora_apply(nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr), LORA_ERR_INVALID_ARGUMENT,
           "apply: ctx NULL");
    expect(lora_shrink_group(nullptr, 1, mods, xs, nullptr), LORA_ERR_INVALID_ARGUMENT, "shrink_group: ctx NULL");
    expect(lora_expand_group(nullptr, 1, mods, ys, nullptr), LORA_ERR_INVALID_ARGUMENT, "expand_group: ctx NULL");
    expect(lora_apply_group(nullptr, 1, mods, xs, ys, nullptr, 0, nullptr), LORA_ERR_INVALID_ARGUMENT,
           "apply_group: ctx NULL");
    expect(lora_apply_group_fused(nullptr, 1, mods, xs, ys, nullptr, 0, nullptr), LORA_ERR_INVALID_ARGUMENT,
           "apply_group_fused: ctx NULL");
    expect(lora_apply_group_noalloc(nullptr, 1, mods, xs, ys, nullptr, 0, nullptr),
           LORA_ERR_INVALID_ARGUMENT, "apply_group_noalloc: ctx NULL");
    expect(lora_get_device_flags(nullptr, &flags), LORA_ERR_INVALID_ARGUMENT, "flags: ctx NULL");
    expect(lora_get_stats(nullptr, &st), LORA_ERR_INVALID_ARGUMENT, "stats: ctx NULL");
    expect(lora_profile_begin(nullptr, 4), LORA_ERR_INVALID_ARGUMENT, "profile_begin: ctx NULL");
    expect(lora_profile_end(nullptr, &pr), LORA_ERR_INVALID_ARGUMENT, "profile_end: ctx NULL");
    expect(lora_slots_destroy(nullptr), LORA_OK, "destroy: NULL accepted");
    // status strings for every code, and one unknown
    for (int s = 1; s >= -10; --s)
        if (lora_status_string(s) == nullptr || lora_status_string(s)[0] == 0) {
            std::printf("FAIL status string %d\n", s);
            ++failures;
        }
    std::printf("failures: %d\n", failures);
    return failures;
}
