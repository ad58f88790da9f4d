/*
 * fa2.h -- C ABI of the FlashAttention-2 library for AMD Instinct MI355X (gfx950),
 * libfa2.so: the forward pass (one-pass and split-KV), the merge of partial
 * results, and the backward pass.
 *
 * Operation (the forward entry points): exact scaled dot-product attention, forward only,
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
 * Head dimension d: 32, 64 or 128 everywhere; 96 and 256 also for every bf16 / fp16
 * entry point (forward, backward, merge; not fa2_fwd_f32).  The d = 256 kernels run
 * one wavefront per SIMD; d = 96 rows take d = 128 rows in on-chip memory (the extra
 * columns are neither loaded nor read).
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

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa2_status {
    FA2_OK = 0,
    FA2_ERR_NULL = 1,            /* a tensor pointer is NULL */
    FA2_ERR_DIM = 2,             /* B, H, Lq or Lk <= 0, an element count overflows int64, the
                                    grid does not fit, or (Lk + 64) * d * element size of one
                                    head's K exceeds 2^31 - 1 bytes */
    FA2_ERR_UNSUPPORTED_D = 3,   /* head dimension d not in {32, 64, 128}, or 96 / 256 for
                                    the bf16/fp16 entry points and the merge */
    FA2_ERR_ARG = 4,             /* causal not 0 or 1, scale not finite or <= 0, num_splits or
                                    dropout_p out of range */
    FA2_ERR_ALIGN = 5,           /* a tensor pointer is not 16-byte aligned */
    FA2_ERR_DEVICE = 6,          /* no usable HIP device, or the device is not gfx950 */
    FA2_ERR_LAUNCH = 7,          /* the kernel launch was refused by the runtime */
    FA2_ERR_WORKSPACE = 8,       /* workspace NULL or smaller than fa2_splitkv_workspace_bytes /
                                    fa2_bwd_workspace_bytes */
    FA2_ERR_SCRATCH = 9          /* fa2_fwd_splitkv_static: the partial results need more than
                                    FA2_STATIC_SCRATCH_BYTES */
} fa2_status;

/*
 * Forward pass with bfloat16 q, k, v, o: the operation of "Triton内核实战：手写
 * FlashAttention-2，优化长序列GPU内存瓶颈", section "标准注意力为何是内存瓶颈" (O =
 * softmax(Q K^T scale) V), with the host interface of its section "Host端包装器与内核
 * 启动" (Q, K, V, causal in; O and the per-row statistic out), computed by the
 * recurrence of "FlashAttention 怎么做? online softmax 怎么更新?", section "推导 / 关键
 * 公式".  Products run on bf16 matrix cores with
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
 * Forward pass with fp16 (IEEE half) q, k, v, o: the same kernel on fp16 matrix
 * cores, probabilities rounded to fp16 and o stored in fp16, both round to
 * nearest even (the fp16 store of "Triton内核实战：手写FlashAttention-2，优化长序列GPU
 * 内存瓶颈", section "流式注意力核心内核").  Same arguments and rules as fa2_fwd.
 */
int fa2_fwd_f16(const void *q, const void *k, const void *v, void *o, float *lse,
                int B, int H, int Lq, int Lk, int d, float scale, int causal, void *stream);

/*
 * Forward pass with fp32 q, k, v, o: fp32 matrix-core products and fp32 state
 * throughout (no reduced-precision step).  The operation of fa2_fwd, i.e. the
 * attention of "Triton内核实战：手写FlashAttention-2，优化长序列GPU内存瓶颈", section
 * "标准注意力为何是内存瓶颈", on fp32 inputs.  Same arguments and rules as fa2_fwd.
 */
int fa2_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                int B, int H, int Lq, int Lk, int d, float scale, int causal, void *stream);

/*
 * Forward pass over a window of keys around each query (sliding-window / local
 * attention), bf16: key j is visible to query i iff
 *     (window_left  < 0  or  j >= i - window_left)   and
 *     (window_right < 0  or  j <= i + window_right),
 * so (-1, -1) is full attention, (-1, 0) the causal mask of fa2_fwd, and
 * (W - 1, 0) a causal window of W keys.  "Flash Attention 全解析（上）", section
 * 5.3, names sliding-window attention as a variant the family goes on to support;
 * the pages give no formula, and this window is the reading adopted.  Only the K/V
 * blocks that hold a visible key of some row of a Q block are visited, so the work
 * scales with the window, not with Lk.  A row that sees no key (possible only with
 * a window, e.g. Lq > Lk) gets o = 0 and lse = -inf.  Same arguments, precision,
 * layout and error rules as fa2_fwd otherwise.
 */
int fa2_fwd_window(const void *q, const void *k, const void *v, void *o, float *lse,
                   int B, int H, int Lq, int Lk, int d, float scale, int window_left, int window_right,
                   void *stream);

/* fa2_fwd_window on fp16 q, k, v, o (precision as fa2_fwd_f16): the window variant of
 * "Flash Attention 全解析（上）", section 5.3. */
int fa2_fwd_window_f16(const void *q, const void *k, const void *v, void *o, float *lse,
                       int B, int H, int Lq, int Lk, int d, float scale, int window_left, int window_right,
                       void *stream);

/*
 * Forward pass with dropout on the attention probabilities, bf16.  "Flash
 * Attention 全解析（上）", section 2.1.2, lists dropout among the steps fused into
 * the one pass over a score block, without fixing a generator; this is the reading
 * adopted:
 *     o = (P * Z * 256 / t) V,   P = softmax(scale q k^T) (causal mask as fa2_fwd)
 * with the keep mask Z[b, h, i, j] = [u < t], t = round(256 (1 - dropout_p)) (ties
 * to even, clamped to 1..256), and u = byte (j mod 4) of output word (i mod 4) of
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) at counter
 * (j / 4, i / 4, b * H + h, offset) and key (seed & 0xffffffff, seed >> 32).
 * The keep probability is t / 256 (dropout_p is quantised to multiples of 1/256).
 * lse is the logsumexp of the scores WITHOUT dropout, as fa2_fwd writes it.  The
 * same (seed, offset) must be passed to fa2_bwd_dropout for the gradients; a caller
 * that draws a fresh mask per step changes offset (or seed).
 *   dropout_p : in [0, 1); 0 keeps everything (o as fa2_fwd, to rounding)
 * FA2_ERR_ARG also for dropout_p outside [0, 1) or NaN.  Same arguments, precision,
 * layout and error rules as fa2_fwd otherwise.
 */
int fa2_fwd_dropout(const void *q, const void *k, const void *v, void *o, float *lse,
                    int B, int H, int Lq, int Lk, int d, float scale, int causal,
                    double dropout_p, uint64_t seed, uint32_t offset, void *stream);

/* fa2_fwd_dropout on fp16 q, k, v, o (the same keep mask; precision as fa2_fwd_f16): the
 * fused dropout of "Flash Attention 全解析（上）", section 2.1.2. */
int fa2_fwd_dropout_f16(const void *q, const void *k, const void *v, void *o, float *lse,
                        int B, int H, int Lq, int Lk, int d, float scale, int causal,
                        double dropout_p, uint64_t seed, uint32_t offset, void *stream);

/*
 * Split-KV forward (FlashDecoding): the same result as fa2_fwd, computed in two
 * stages on `stream` ("Flash Attention 全解析（上）", section 4.3).
 *
 *  1. Every Q block's visible K/V blocks are cut into num_splits contiguous,
 *     near-equal ranges, and each (Q block, range) pair is an independent
 *     work-group, so short-Lq or few-head problems still fill the GPU (the
 *     Q-length-1 problem of section 4.1 of that page).  Each work-group runs the
 *     fa2_fwd recurrence over its range only and writes, per query row, the
 *     partial result normalised by its own sum, O_s (fp32, [d]), and its
 *     logsumexp L_s (fp32, natural log).  A row that sees no key of its range
 *     gets L_s = -inf and its O_s is left unwritten.
 *  2. A merge kernel (fa2_merge_partials below) combines the partials of every
 *     row.
 *
 * With Lq <= 4 (decoding) stage 1 runs a kernel for a few query rows instead: one
 * work-group per (b, h, range) streams the range's K and V rows into registers and
 * takes the dot products and the weighted sum of V on the vector ALU in fp32 (the
 * probabilities are not rounded to bf16 there); the partials have the same form.
 *
 * Arguments as fa2_fwd, plus
 *   num_splits     : number of K/V ranges, 1..FA2_MAX_SPLITS; 0 picks a count
 *                    for the current device (fa2_splitkv_num_splits).  Ranges of
 *                    a Q block with fewer K/V blocks than splits may be empty;
 *                    such work-groups only mark their rows L_s = -inf.
 *   workspace      : device memory of at least fa2_splitkv_workspace_bytes(...)
 *                    bytes, 16-byte aligned, owned by the caller; the call
 *                    overwrites it and needs no prior contents.  Calls that run
 *                    at the same time need separate workspaces.
 *   workspace_bytes: its size; too small -> FA2_ERR_WORKSPACE, nothing launched.
 * A split count of 1 (given, or chosen for num_splits == 0) runs fa2_fwd's
 * one-pass kernel and leaves the workspace untouched.
 */
#define FA2_MAX_SPLITS 128

int fa2_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                    int B, int H, int Lq, int Lk, int d, float scale, int causal,
                    int num_splits, void *workspace, size_t workspace_bytes, void *stream);

/*
 * fa2_fwd_splitkv without a workspace and without any allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The partial results live in
 * a static device array of the library, FA2_STATIC_SCRATCH_BYTES bytes on every
 * device the library runs on, held until the process ends (its address on a
 * device is looked up on the first call there).  bf16 only; the same kernels,
 * split count, results and errors as fa2_fwd_splitkv, plus:
 *   FA2_ERR_SCRATCH : the partials (fa2_splitkv_workspace_bytes for the same
 *                     arguments) exceed FA2_STATIC_SCRATCH_BYTES; nothing is
 *                     launched.  With num_splits > 0 this is decided before any
 *                     HIP call.  A split count of 1 needs no scratch.
 * All calls on one device share that device's array and nothing else orders
 * them: calls that overlap in time on one device (two streams, two host
 * threads) race on it and may return wrong results.  Serialise them, or use
 * fa2_fwd_splitkv with a workspace per stream.  The array needs no clearing: a
 * call writes every partial it reads.
 */
#define FA2_STATIC_SCRATCH_BYTES (32u * 1024u * 1024u)

int fa2_fwd_splitkv_static(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int H, int Lq, int Lk, int d, float scale, int causal, int num_splits,
                           void *stream);

/* fa2_fwd_splitkv on fp16 q, k, v, o (the same workspace; o rounded to fp16, nearest
 * even, by the merge): the split-KV forward of "Flash Attention 全解析（上）", section
 * 4.3. */
int fa2_fwd_splitkv_f16(const void *q, const void *k, const void *v, void *o, float *lse,
                        int B, int H, int Lq, int Lk, int d, float scale, int causal,
                        int num_splits, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Workspace bytes fa2_fwd_splitkv needs for the per-range partial results of the
 * split-KV forward ("Flash Attention 全解析（上）", section 4.3) for these sizes:
 * num_splits * B * H * Lq
 * rows of (d + 1) fp32 values, laid out as the partial outputs
 * [num_splits, B, H, Lq, d] followed (at a 256-byte boundary) by the partial
 * logsumexps [num_splits, B, H, Lq].  num_splits == 0 resolves as in
 * fa2_fwd_splitkv (so it needs Lk, causal and the current device).  Returns 0
 * for sizes fa2_fwd_splitkv would reject.
 */
size_t fa2_splitkv_workspace_bytes(int B, int H, int Lq, int Lk, int d, int causal, int num_splits);

/*
 * The split count num_splits == 0 stands for (the split of the K/V sequence that
 * fills the device when Q is short, "Flash Attention 全解析（上）", sections 4.1 and
 * 4.3): the fewest ranges that give every
 * compute unit of the current device one (Q block, range) work-group, or two
 * when causal (Q blocks then differ in length), with at least 8 K/V blocks per
 * range and at most FA2_MAX_SPLITS ranges; 1 when the Q blocks alone fill the
 * device.  With Lq <= 4: the fewest ranges that give every compute unit two
 * (b, h, range) work-groups, with at least 256 keys per range.  Returns 1 if the
 * device cannot be queried.
 */
int fa2_splitkv_num_splits(int B, int H, int Lq, int Lk, int d, int causal);

/*
 * Merge n_parts partial attention results of the same queries over disjoint
 * key sets into the result over their union: for every row r,
 *     M   = max_s L_s[r]
 *     W   = sum_s exp(L_s[r] - M)
 *     O[r]   = sum_s exp(L_s[r] - M) O_s[r] / W      (rounded to bf16, nearest even)
 *     LSE[r] = M + ln W
 * i.e. LSE = ln sum_s exp(L_s) and O = sum_s exp(L_s - LSE) O_s, the combine of
 * two normalised halves in "FlashAttention 怎么做? online softmax 怎么更新?",
 * follow-up question "多卡(ring attention)怎么合并两段结果?", applied to n parts; it is
 * also the global rescaling of section 4.3 of "Flash Attention 全解析（上）".
 * Parts with L_s = -inf contribute nothing and their O_s is not read; a row
 * whose parts are all -inf gets O = 0 and LSE = -inf.
 *   o_parts   : fp32 [n_parts, rows, d]    lse_parts : fp32 [n_parts, rows]
 *   o         : bf16 [rows, d]             lse       : fp32 [rows]
 *   n_parts 1..FA2_MAX_SPLITS, rows >= 1, d in {32, 64, 96, 128, 256}; device pointers,
 *   16-byte aligned, caller-owned; outputs must not overlap inputs.
 */
int fa2_merge_partials(const float *o_parts, const float *lse_parts, int n_parts, int64_t rows,
                       int d, void *o, float *lse, void *stream);

/* fa2_merge_partials writing fp16 o (round to nearest even): the combine of
 * "FlashAttention 怎么做? online softmax 怎么更新?", follow-up question "多卡(ring
 * attention)怎么合并两段结果?". */
int fa2_merge_partials_f16(const float *o_parts, const float *lse_parts, int n_parts, int64_t rows,
                           int d, void *o, float *lse, void *stream);

/*
 * Backward pass (gradients) of fa2_fwd, bf16.  Given the forward's inputs, its
 * outputs o and lse, and dout = dL/dO, computes dq = dL/dQ, dk = dL/dK and
 * dv = dL/dV of the same attention (same scale, same causal mask):
 *
 *     P    = exp(scale * Q K^T - LSE)             (masked keys: 0)
 *     D_i  = sum_t dout_it o_it
 *     dV   = P^T dout          dP = dout V^T       dS = P * (dP - D)
 *     dQ   = scale * dS K      dK = scale * dS^T Q
 *
 * The score and probability blocks are rebuilt from q, k and lse instead of
 * being stored by the forward ("FlashAttention 怎么做? online softmax 怎么更新?",
 * section "Recomputation"); the formulas are the derivative of the forward
 * definition.  Products run on bf16 matrix cores with fp32 accumulation; P and
 * dS are rounded to bf16 (nearest even) before they enter a product; dq, dk, dv
 * are rounded to bf16 (nearest even).  dQ is computed by a pass of its own over
 * the key blocks rather than accumulated with atomics, so results are
 * run-to-run bitwise identical.
 *   q, k, v, o, dout : bf16 device pointers; q, o, dout [B, H, Lq, d], k, v [B, H, Lk, d]
 *   lse              : fp32 [B, H, Lq], as written by fa2_fwd for these q, k, v
 *   dq, dk, dv       : bf16 outputs, shapes of q, k, v; completely overwritten (keys
 *                      that no query sees under the causal mask get 0)
 *   workspace        : device memory of at least fa2_bwd_workspace_bytes(B, H, Lq)
 *                      bytes, 16-byte aligned, caller-owned; overwritten, needs no
 *                      prior contents; concurrent calls need separate workspaces
 * Other arguments, layout and error rules as fa2_fwd; additionally
 * FA2_ERR_WORKSPACE for a missing or too small workspace.  Outputs must not
 * overlap inputs or each other (not checked).
 */
int fa2_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
            void *dq, void *dk, void *dv, int B, int H, int Lq, int Lk, int d, float scale, int causal,
            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward pass of fa2_fwd_f16: fp16 q, k, v, o, dout, dq, dk, dv (fp16 matrix
 * cores, P and dS rounded to fp16, outputs fp16, round to nearest even); the
 * recomputation of "FlashAttention 怎么做? online softmax 怎么更新?", section
 * "Recomputation".  Same arguments and rules as fa2_bwd.
 */
int fa2_bwd_f16(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
                void *dq, void *dk, void *dv, int B, int H, int Lq, int Lk, int d, float scale, int causal,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward pass of fa2_fwd_dropout: the gradients of o = (P * Z * 256 / t) V with
 * the keep mask Z of (dropout_p, seed, offset) -- pass exactly the values given to
 * the forward that wrote o and lse; the mask is drawn again, not stored.  With
 * A = P * Z * 256 / t:
 *     dv = A^T dout,   dP = (dout v^T) * Z * 256 / t,   D = rowsum(dout * o),
 *     dS = P * (dP - D),   dq = scale dS k,   dk = scale dS^T q
 * (the derivative of that forward; the reading is described at fa2_fwd_dropout;
 * dropout fused into the pass over a score block as in "Flash Attention 全解析（上）",
 * section 2.1.2, the probabilities rebuilt as in "FlashAttention 怎么做? online
 * softmax 怎么更新?", section "Recomputation").
 * Same arguments, precision, workspace and error rules as fa2_bwd; FA2_ERR_ARG
 * also for dropout_p outside [0, 1).
 */
int fa2_bwd_dropout(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
                    void *dq, void *dk, void *dv, int B, int H, int Lq, int Lk, int d, float scale, int causal,
                    double dropout_p, uint64_t seed, uint32_t offset, void *workspace, size_t workspace_bytes,
                    void *stream);

/* fa2_bwd_dropout on fp16 data (the backward of fa2_fwd_dropout_f16; dropout as in
 * "Flash Attention 全解析（上）", section 2.1.2). */
int fa2_bwd_dropout_f16(const void *q, const void *k, const void *v, const void *o, const float *lse,
                        const void *dout, void *dq, void *dk, void *dv, int B, int H, int Lq, int Lk, int d,
                        float scale, int causal, double dropout_p, uint64_t seed, uint32_t offset,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward pass of fa2_fwd_window (the window of "Flash Attention 全解析（上）",
 * section 5.3, with the recomputation of "FlashAttention 怎么做? online softmax 怎么
 * 更新?", section "Recomputation"): the gradients of attention over the key
 * window (window_left, window_right) of fa2_fwd_window, from its o and lse.
 * Rows that see no key contribute nothing (their o = 0, D = 0, P = 0); keys no
 * row sees get dk = dv = 0.  Same arguments and rules as fa2_bwd otherwise.
 */
int fa2_bwd_window(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
                   void *dq, void *dk, void *dv, int B, int H, int Lq, int Lk, int d, float scale,
                   int window_left, int window_right, void *workspace, size_t workspace_bytes, void *stream);

/* fa2_bwd_window on fp16 data (the backward of fa2_fwd_window_f16; "Flash Attention
 * 全解析（上）", section 5.3). */
int fa2_bwd_window_f16(const void *q, const void *k, const void *v, const void *o, const float *lse,
                       const void *dout, void *dq, void *dk, void *dv, int B, int H, int Lq, int Lk, int d,
                       float scale, int window_left, int window_right, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * Workspace bytes fa2_bwd needs for the per-row statistics its recomputation reads
 * ("FlashAttention 怎么做? online softmax 怎么更新?", section "Recomputation": the
 * saved L, and D = rowsum(dO * O)): lse * log2(e) for the B*H*Lq query rows and,
 * from the next 256-byte boundary, D = rowsum(dout * o) for the same rows, both
 * fp32.  Returns 0 for sizes that do not fit.
 */
size_t fa2_bwd_workspace_bytes(int B, int H, int Lq);

/* Static English text for a status code (never NULL): the status of the argument
 * checks and launches of the entry points, whose interface is the host wrapper of
 * "Triton内核实战：手写FlashAttention-2，优化长序列GPU内存瓶颈", section "Host端包装器与
 * 内核启动". */
const char *fa2_status_string(int status);

/*
 * Validate arguments of the forward of "Triton内核实战：手写FlashAttention-2，优化长序列
 * GPU内存瓶颈" (section "Host端包装器与内核启动") exactly as fa2_fwd / fa2_fwd_f16 /
 * fa2_fwd_f32 do, without any
 * HIP call.  elem_bytes is 2 (bf16 or fp16) or 4 (fp32).  Returns the status those
 * entry points would return before launching.
 */
int fa2_check_args(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   int B, int H, int Lq, int Lk, int d, float scale, int causal, int elem_bytes);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */
