/*
 * fa2.h -- C ABI of the FlashAttention-2 forward library for AMD Instinct MI355X
 * (gfx950), libfa2.so.
 *
 * Operation (both entry points): exact scaled dot-product attention, forward only,
 * with a per-row logsumexp, for every (batch b, head h, query row i):
 *
 *     s_ij  = scale * (q_i . k_j)            for keys j visible to i
 *     O_i   = sum_j softmax_j(s_i) * v_j
 *     LSE_i = ln( sum_j exp(s_ij) )          (natural log, over visible keys)
 *
 * The problem statement O = softmax(QK^T / sqrt(d)) V is the one of
 * "Triton内核实战：手写FlashAttention-2，优化长序列GPU内存瓶颈", section
 * "标准注意力为何是内存瓶颈", and of "新年一定要学会FlashAttention! FlashAttention极简
 * 教程与实现", section "背景".  The per-row logsumexp L = m + log(l) kept for the
 * backward pass is the one of "FlashAttention 怎么做? online softmax 怎么更新?",
 * section "FlashAttention-2 改了什么", stored as an fp32 [B, H, Lq] buffer as in
 * the Triton page's host wrapper (section "Host端包装器与内核启动").
 *
 * The result is computed by the FlashAttention-2 forward: Q blocks on the outside,
 * K/V blocks on the inside, online softmax with running max and sum, a single
 * division by the row sum after the last K/V block, no score or probability
 * matrix in device memory ("FlashAttention-2 算法架构升级：减少非矩阵乘 FLOPs 与
 * Q-loop 顺序调优", sections 一.2 and 二.2).
 *
 * Causal mask: key j is visible to query i iff j <= i (top-left alignment; the
 * same as bottom-right alignment when Lq == Lk).  Every query row sees key 0, so
 * no row is empty.  Key blocks that are masked for every row of a Q block are
 * skipped ("FlashAttention 怎么做?", section "FlashAttention-2 改了什么").
 *
 * Layout: every tensor is dense, row-major, without strides:
 *     q, o   [B, H, Lq, d]      k, v   [B, H, Lk, d]      lse   [B, H, Lq]  fp32
 * o has the element type of q.  All pointers are DEVICE pointers on the current
 * HIP device and must be 16-byte aligned.
 *
 * Ownership: the caller allocates and owns every buffer.  q, k, v are read only;
 * o and lse are completely overwritten (every row, also for ragged Lq).  The
 * library allocates nothing, keeps no per-call state and never synchronises: the
 * work is enqueued on `stream` (a hipStream_t; NULL means the default stream) and
 * the call returns.  Calls may be made from several host threads.
 *
 * Errors: every entry point returns an fa2_status.  All argument checks run
 * before any HIP call, so a rejected call touches no device state.  A launch that
 * the runtime refuses returns FA2_ERR_LAUNCH.  Faults during execution surface at
 * the caller's next synchronisation with the stream, as for any asynchronous work.
 * o and lse must not overlap q, k, v or each other (not checked).
 */
#ifndef FA2_H
#define FA2_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa2_status {
    FA2_OK = 0,
    FA2_ERR_NULL = 1,            /* a tensor pointer is NULL */
    FA2_ERR_DIM = 2,             /* B, H, Lq or Lk <= 0, or an element count overflows int64 */
    FA2_ERR_UNSUPPORTED_D = 3,   /* head dimension d not in {64, 128} */
    FA2_ERR_ARG = 4,             /* causal not 0 or 1, or scale not finite or <= 0 */
    FA2_ERR_ALIGN = 5,           /* a tensor pointer is not 16-byte aligned */
    FA2_ERR_DEVICE = 6,          /* no usable HIP device, or the device is not gfx950 */
    FA2_ERR_LAUNCH = 7           /* the kernel launch was refused by the runtime */
} fa2_status;

/*
 * Forward pass with bfloat16 q, k, v, o.  Products run on bf16 matrix cores with
 * fp32 accumulation; the running max m, running sum l and the unnormalised output
 * stay fp32; the probabilities are rounded to bf16 (round to nearest even) before
 * they multiply V; o is rounded to bf16 with round to nearest even; lse is fp32.
 *   q, k, v, o : bf16 device pointers (uint16 bit patterns), layouts above.
 *   lse        : fp32 device pointer, [B, H, Lq].
 *   scale      : multiplies q . k before the softmax (usually 1/sqrt(d)); finite, > 0.
 *   causal     : 0 or 1.
 *   stream     : hipStream_t to enqueue on.
 */
int fa2_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
            int B, int H, int Lq, int Lk, int d, float scale, int causal, void *stream);

/*
 * Forward pass with fp32 q, k, v, o: fp32 matrix-core products and fp32 state
 * throughout (no reduced-precision step).  Same arguments and rules as fa2_fwd.
 */
int fa2_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                int B, int H, int Lq, int Lk, int d, float scale, int causal, void *stream);

/* Static English text for a status code (never NULL). */
const char *fa2_status_string(int status);

/*
 * Validate arguments exactly as fa2_fwd / fa2_fwd_f32 do, without any HIP call.
 * elem_bytes is 2 (bf16) or 4 (fp32).  Returns the status those entry points
 * would return before launching.
 */
int fa2_check_args(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   int B, int H, int Lq, int Lk, int d, float scale, int causal, int elem_bytes);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */
