/*
 * park_clocks.h - measurement-only entry points of libpark_clocks.so, the build of libpark
 * whose attention kernel carries per-item clock stamps (compiled with PARK_ATTN_CLOCKS).
 * libpark.so, the product library, exports neither function and stamps nothing.
 *
 * Every other entry point of libpark_clocks.so is the one declared in park.h, with the same
 * behaviour; the stamped attention kernel adds four shader-clock reads (s_memtime) and one
 * 40-byte store per item to the work of park_block_sparse_attn (64-token query blocks).
 *
 * Record layout: five 64-bit words per item of the last park_block_sparse_attn call, at
 * word 5 i for item i = (B H row) * kRanges + key range, kRanges = 4:
 *   [0] clock at the item's start, [1] before its tile loop, [2] after the loop,
 *   [3] after its output stores, [4] (workgroup index << 32) | tiles in the item.
 * Items with no tile, and items past the record's capacity, leave their five words as they
 * were (zero after the library is loaded).  The clock is the shader clock of the XCD the
 * item ran on: differences within one item or one workgroup are cycles; stamps of different
 * XCDs are not comparable.
 */
#ifndef PARK_CLOCKS_H
#define PARK_CLOCKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define PARK_CLOCKS_API __attribute__((visibility("default")))
#else
#define PARK_CLOCKS_API
#endif

/* Capacity of the record in 64-bit words (5 per item). */
PARK_CLOCKS_API size_t park_attn_clock_words(void);

/* Copy the first `words` words of the record to `host` (host memory, caller-owned, at least
 * 8 * words bytes), synchronously on the current device.  Returns PARK_OK, PARK_ERR_INVALID
 * (host NULL or words above the capacity) or PARK_ERR_HIP (the copy failed). */
PARK_CLOCKS_API int park_attn_clock_read(void* host, size_t words);

#ifdef __cplusplus
}
#endif

#endif /* PARK_CLOCKS_H */
