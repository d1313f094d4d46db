/*
 * svdq_bench.h -- measurement entry point of libsvdq.so (not part of the layer's data path).
 *
 * The roofline of the W4A4 product is priced against the dense int8 matrix-core peak of the
 * chip (256 CUs x 2.4 GHz x 8192 int8 operations per clock and CU). A loaded MI355X runs below
 * its peak clock, so the measurement also needs the rate a pure matrix-core loop reaches and the
 * clock it runs at; and the rescale design of the W4A4 kernel rests on the relative cost of the
 * float32 matrix and vector units. svdq_bench_unit_peak provides these figures.
 */
#ifndef SVDQ_BENCH_H_
#define SVDQ_BENCH_H_

#ifdef __cplusplus
extern "C" {
#endif

enum svdq_bench_kind {
  SVDQ_BENCH_MFMA_I8_32X32X32 = 0,    /* v_mfma_i32_32x32x32_i8: 2*32*32*32 int8 ops each */
  SVDQ_BENCH_MFMA_BF16_32X32X16 = 1,  /* v_mfma_f32_32x32x16_bf16: 2*32*32*16 flops each */
  SVDQ_BENCH_MFMA_F32_32X32X1_2B = 2, /* v_mfma_f32_32x32x1_2b_f32: two 32x32 outer products, 4096 flops */
  SVDQ_BENCH_VALU_FMA_F32 = 3,        /* v_fma_f32 on 64 lanes: 128 flops each */
  SVDQ_BENCH_MIX_I8_FMA = 4           /* per 16 instructions: 16 int8 MFMAs as above plus 256
                                         independent v_fma_f32 (the W4A4 rescale's proportion) */
};

/* Launch `blocks` blocks of 256 threads (4 waves) on `stream`; every wave issues
 * iters * 16 instructions of the chosen kind in four independent chains (VALU: iters * 64 FMAs
 * in sixteen chains; MIX: iters * 16 MFMAs and iters * 256 FMAs, interleaved) and touches no
 * memory in its loop. Block b writes clocks[2b] = shader-clock
 * cycles (s_memtime) and clocks[2b + 1] = 100 MHz real-time ticks (s_memrealtime) elapsed
 * around its loop. clocks: device memory, 2*blocks uint64; sink: device memory, 256 int32, never
 * written in practice (it keeps the results live). Asynchronous; allocates nothing.
 * Returns 0, -1 (NULL pointer), -2 (blocks outside [1, 2^20] or iters outside [1, 2^24]),
 * -4 (unknown kind) or -6 (launch failed). */
int svdq_bench_unit_peak(int kind, int blocks, int iters, unsigned long long* clocks, int* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_BENCH_H_ */
