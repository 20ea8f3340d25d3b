/*
 * tj2_measure.h -- C ABI of libtj2_measure, the measurement helpers that the
 * benchmark times beside the products.  They are not part of the quantized
 * linear layer and live in a library of their own (libtj2_measure.so); the
 * product library libtj2.so exports none of them.
 */
#ifndef TJ2_MEASURE_H_
#define TJ2_MEASURE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The achievable dense f16 MFMA rate of the part.  Runs `workgroups`
 * workgroups of 256 threads (4 waves); each wave runs `iters` rounds of four
 * independent v_mfma_f32_32x32x16_f16 accumulation chains on register
 * operands (every element 0.0625, so each thread's result, written to
 * out[workgroup * 256 + thread], is 0.25 * iters exactly).  Work: workgroups *
 * 4 * iters * 4 * 32768 flops; the caller times the call on its stream.
 * out: device, workgroups * 256 floats, caller-owned.  Returns 0, 1 (NULL out,
 * workgroups outside [1, 2^20] or iters outside [1, 2^20]; nothing enqueued)
 * or 4 (launch error).
 */
int32_t tj2_mfma_peak_probe(int64_t workgroups, int32_t iters, float* out, void* stream);

/*
 * Where the B operand of a packed product is decoded: the product kernel's
 * inner loop without global memory (per 128-K chunk: barrier, B stage written
 * to LDS, barrier, 8 A fragments decoded in registers per wave, 32
 * v_mfma_f32_32x32x16_f16 per wave), with B decoded once per workgroup into
 * f16 in LDS (packed_b == 0) or staged packed (E2M1 codes + E4M3 scales) and
 * decoded by every wave after its LDS reads (packed_b != 0).  Synthetic data,
 * changed every chunk.  `workgroups` workgroups of 512 threads; work:
 * workgroups * 8 * iters * 32 * 32768 flops.  out: device, workgroups * 512
 * floats (finite values; their content is not meaningful).  Returns 0, 1 (bad
 * arguments; nothing enqueued) or 4 (launch error).
 */
int32_t tj2_decode_probe(int32_t packed_b, int64_t workgroups, int32_t iters, float* out, void* stream);

/*
 * The access pattern of the OsciReset pass (nsrc = 5 reads, ndst = 4 writes,
 * 36 B per element) or of the fused master-weight pass (nsrc = 7, ndst = 6,
 * 52 B per element) without their arithmetic: element-wise over n fp32
 * elements (the first n - n % 8), 8 consecutive elements per thread, every
 * load issued before the stores, dst[i][e] = src[i][e] + src[nsrc - 1][e].
 * src, dst: host arrays of device pointers (16-byte aligned, n floats each,
 * caller-owned; the destinations may not overlap the sources).  Returns 0, 1
 * (NULL or misaligned pointer, n outside [8, 2^36], or another nsrc / ndst
 * pair; nothing enqueued) or 4 (launch error).
 */
int32_t tj2_stream_probe(const float* const* src, int32_t nsrc, float* const* dst, int32_t ndst, int64_t n,
                         void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TJ2_MEASURE_H_ */
