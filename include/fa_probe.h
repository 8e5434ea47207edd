/*
 * fa_probe.h -- C ABI of libfa_probe.so: issue-rate probes of one SIMD of
 * the MI355X (gfx950).  Measurement support for the attention kernels'
 * roofline, not part of the attention path.
 *
 * The FlashAttention-4 article («Оптимизируйте производительность с
 * FlashAttention-4», paragraph 3) attributes the forward's cost on Blackwell
 * to the exponential unit rather than the tensor cores, and computes part of
 * the exponentials with ordinary FMA instructions.  Whether either holds on
 * this chip depends on what a v_exp_f32 costs a SIMD next to a v_fma_f32,
 * the packing and maximum instructions of the softmax, and the matrix
 * instructions, and on how they overlap; these probes measure exactly that.
 */
#ifndef FA_PROBE_H_
#define FA_PROBE_H_

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_probe_rates -- one timing launch.
 *   a, b    instruction bodies (ids as in fa_probe_rates.hip: 1 v_fma_f32,
 *           2 v_exp_f32, 3 exp + fma interleaved, 4 v_cvt_pk_fp8_f32,
 *           5 v_maximum3_f32, 6 v_add_f32, 7 f8 MFMA 32x32x64, 8 bf16 MFMA
 *           32x32x16, 9 f8 MFMA with exp / fma, 10 bf16 MFMA with exp and
 *           fma, 11 fma -> exp -> add chains, 12 bf16 MFMA and 13 f8 MFMA
 *           on operands from `data`, 2 A and 2 B fragments paired in
 *           turn, 14 v_dot2c_f32_bf16, 15 v_mov_b64, 16 v_cvt_pk_bf16_f32,
 *           17 / 18 / 19 bf16 MFMA each followed by 4 v_add_f32 / 4
 *           v_dot2c_f32_bf16 / 4 v_mov_b64 in the same wave, 20
 *           v_cvt_scalef32_pk_fp8_f32, 21 the bf16 forward's issue slot
 *           (scores MFMA, two v_fma_f32 -> v_exp_f32, P V MFMA into
 *           accumulation registers, v_cvt_pk_bf16_f32 and two v_add_f32),
 *           22 ds_read_b128 at the bf16 forward's K fragment addresses, 23
 *           ds_read_b64_tr_b16 at its V fragment addresses, 24
 *           ds_read_b64_tr_b16 at consecutive 8-byte units, 25 the
 *           FMA-pipe exponential of fa_fwd_fp8_exp2_fma (16 per round,
 *           eight vector instructions each), 26 body 21 with its vector
 *           work pipelined across slots (the FMAs of pair i + 1 and the
 *           exponentials of pair i after the first MFMA, the pack and
 *           sums of pair i - 1 after the second), 27 16 LDS-DMA tile
 *           copies (buffer_load_dwordx4 ... lds, 1 KB each) from `data`
 *           into the wave's slice of the LDS reserve, 28 4 x (bf16 MFMA +
 *           one such copy), 29 body 21 with one such copy after its first
 *           MFMA (27 to 29 leave at most 8 copies in flight per round); b
 *           may also be 0, idle, and must be for bodies 12, 13, 17 to 19
 *           and 21 to 29).
 *   waves   waves per workgroup, 4..16, a multiple of 4 (one workgroup per
 *           CU, so waves / 4 waves on each SIMD; bodies 22 to 24 read the
 *           workgroup's 96 KiB LDS reserve, shared by its waves).
 *   na      the first 4 * na waves run body a, the others body b.
 *   iters   rounds of the body per wave, >= 1.
 *   grid    workgroups (the CU count for one per CU).
 *   out     device, caller-owned, grid * waves * 3 uint64 (written): per
 *           wave in (workgroup, wave) order, shader-clock cycles between the
 *           two clock reads, 100 MHz reference ticks over the same span, and
 *           the wave's HW_ID register (SIMD in bits 5:4).
 *   data    device, 512 entries of 32 bytes, 32-byte aligned (read only):
 *           operand values of bodies 12 and 13 (lane l, fragment j reads
 *           entries (l + 64 j) % 512 and (l + 64 j + 256) % 512) and the
 *           copy source of bodies 27 to 29; may be NULL for the others.
 *   stream  hipStream_t or NULL; one kernel is enqueued.
 *   Returns 0, 1 for an invalid argument (nothing enqueued), 4 if the
 *   launch failed.
 */
int fa_probe_rates(int a, int b, int waves, int na, int iters, int grid,
                   unsigned long long* out, const void* data, void* stream);

/*
 * fa_probe_read -- one launch that reads `bytes` of device memory once
 * (HBM read bandwidth available to a streaming kernel, the ceiling of the
 * decode path's K/V reads).
 *   src     device, 16-byte aligned, bytes readable (read only; contents
 *           do not matter).
 *   bytes   a positive multiple of 16.
 *   grid    workgroups of 256 threads, >= 1 (each thread keeps eight
 *           16-byte loads in flight, grid-stride over the buffer).
 *   sink    device, caller-owned, grid unsigned words; word g is written
 *           only if workgroup g's threads read a fixed bit pattern.
 *   stream  hipStream_t or NULL; one kernel is enqueued.
 *   Returns 0, 1 for an invalid argument (nothing enqueued), 4 if the
 *   launch failed.
 */
int fa_probe_read(const void* src, unsigned long long bytes, int grid,
                  unsigned* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H_ */
