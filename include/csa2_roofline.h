/*
 * csa2_roofline.h -- measurement helper shipped beside the CSA2 library (in
 * libcsa2_roofline.so, not part of the method): the streaming-read ceiling
 * against which the indexer scan's bandwidth is reported.
 */
#ifndef CSA2_ROOFLINE_H
#define CSA2_ROOFLINE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * csa2roof_stream_read -- enqueue one plain read of `bytes` bytes at device
 * pointer `src` (16-byte aligned, bytes a multiple of 16) by `blocks`
 * workgroups of 256 lanes, grid-stride, 16 bytes per load with the
 * non-temporal hint.  `sink` is a device word written only if the folded data
 * equals a fixed sentinel.  Returns 0, -1 for a bad argument (nothing
 * enqueued), or -5 if the launch failed.  Caller-owned memory and stream.
 */
int csa2roof_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_ROOFLINE_H */
