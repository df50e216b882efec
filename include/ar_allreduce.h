/*
 * ar_allreduce.h -- C ABI of the MI355X sum all-reduce over R rank buffers.
 *
 * One process, one GPU.  R "ranks" are R buffers in the GPU's HBM that stand
 * in for the peer memory a memory-mapped channel would expose (the
 * MemoryChannel of "MSCCL++：让 GPU 通信像 CUDA 一样可编程",
 * infinitensor.com/news/50, section "MemoryChannel": GPU threads load and store
 * the other GPU's memory directly).  One call reduces the R send buffers
 * element by element and writes the sum to all R receive buffers.
 *
 * The call is shaped like the NCCL-compatible collective that the same page
 * describes under "第一层：Collective API" (mscclppAllReduce as a drop-in for
 * ncclAllReduce), with the R rank pointers of the simulated group passed as
 * arrays.  Two protocols from the page's MemoryChannel table are offered:
 *
 *   arProtoLL  low latency: one kernel, flag-carrying 8-byte (or 16-byte)
 *              packets, polled per wavefront; meant for decode-size messages.
 *   arProtoHB  high bandwidth: two-shot reduce-scatter by chunk then
 *              all-gather, 128-bit bulk loads and stores, no flags; meant for
 *              prefill-size messages.  A staged form with a kernel boundary
 *              between the shots is available as an option.
 *
 * Both give the same result: for every element i,
 *     a = x_0[i];  a = a + x_j[i] for j = 1..R-1 (binary32, in this order);
 *     recv_r[i] = a rounded to the element type (round to nearest even),
 * which is one reading of a SUM all-reduce over float/float16/bfloat16, the
 * operations and types admitted by the runtime guards of "SGLang 中的 MSCCL++
 * All-Reduce 基准测试与推理集成指南" (blog.gitcode.com), section 4.3.
 *
 * Errors are return codes; nothing here aborts, throws or prints (except with
 * the environment variable AR_DEBUG=1, which logs rejected calls to stderr).
 * A result of arUnsupported means "use another all-reduce", the fallback the
 * SGLang guide describes when a guard fails (sections 4.3 and 5).
 *
 * All entry points are host functions.  A communicator is used from one host
 * thread and one stream at a time, like an NCCL communicator: its LL packet
 * memory is shared by its calls, so two LL calls of one communicator must not
 * overlap in time.  Several communicators may run at once on different
 * streams.  An LL call needs all of its workgroups resident together, so
 * concurrent kernels that fill the GPU can delay an LL call up to its wait
 * bound (arOptPollTimeoutUs), after which it records arTimeout.
 */
#ifndef AR_ALLREDUCE_H
#define AR_ALLREDUCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AR_VERSION 10200 /* 1.2.0 */
#define AR_MAX_RANKS 32

typedef struct arComm *arComm_t;

/* A hipStream_t, passed as an untyped pointer so that this header does not
 * need the HIP headers.  NULL is the device's null stream. */
typedef void *arStream_t;

typedef enum {
    arSuccess = 0,
    arInvalidArgument = 1, /* a pointer, size, alignment or overlap rule broken */
    arUnsupported = 2,     /* valid request this library does not serve: fall back */
    arInvalidUsage = 3,    /* request exceeds what the communicator was made for */
    arHipError = 4,        /* a HIP runtime call failed */
    arTimeout = 5,         /* an LL packet wait ran out of time (asynchronous) */
    arInternalError = 6
} arResult_t;

typedef enum { arBfloat16 = 0, arFloat16 = 1, arFloat32 = 2 } arDataType_t;

typedef enum { arSum = 0 } arRedOp_t;

/* arProtoAuto picks, per message size, the protocol that arCommTune measured
 * faster (HB where nothing was tuned). */
typedef enum { arProtoLL = 0, arProtoHB = 1, arProtoAuto = 2 } arProtocol_t;

/* Tunables and test hooks, see arCommSetOption.  The launch-shape options
 * are the (workgroups, threads per workgroup) pairs that an auto-tuner would
 * time per message size. */
typedef enum {
    /* LL: longest total wait of one lane for packets, in microseconds
     * (default 2,000,000).  A wait that runs out records arTimeout in the
     * communicator and the kernel finishes without the missing data. */
    arOptPollTimeoutUs = 0,
    /* LL: workgroups per simulated rank; 0 = the built-in default for the
     * rank count and message size (a table measured on MI355X; with only
     * arOptLLThreads set, as many lanes per rank as the default has). */
    arOptLLBlocksPerRank = 1,
    /* HB: workgroups in the grid (rounded to a multiple of nranks, capped by
     * the message's tiles); 0 = one per compute unit. */
    arOptHBBlocks = 2,
    /* HB: 1 = non-temporal loads and stores, 0 = ordinary (cached) ones.
     * -1 (default): the policy the tuner chose for the message size and mode,
     * else 1.  On MI355X ordinary accesses win from a few MiB per rank while
     * the message fits the last-level cache, non-temporal ones above it. */
    arOptHBNonTemporal = 3,
    /* Test hook: LL consumers wait for a flag shifted by this value, which no
     * producer writes when the value is not 0, so every wait times out.
     * Default 0. */
    arOptDebugFlagSkew = 4,
    /* HB: 16-byte vectors each lane handles per rank per step (1, 2 or 4;
     * capped at 2 above 4 ranks and at 1 above 8); 0 = default (1). */
    arOptHBUnroll = 5,
    /* LL: threads per workgroup (64, 128, 256, 512 or 1024; capped at 512
     * above 16 ranks); 0 = the built-in default for the rank count and
     * message size. */
    arOptLLThreads = 6,
    /* HB: threads per workgroup (64 .. 1024, a multiple of 64; capped at 512
     * above 8 ranks and 256 above 16); 0 = default (256, or 128 from 32 ranks). */
    arOptHBThreads = 7,
    /* HB: which elements simulated rank c reduces (its chunk) -- 0: the
     * contiguous c-th of R equal parts, 1: every R-th tile starting at tile c
     * (default; streams all R buffers in address order, which HBM serves
     * faster). */
    arOptHBChunkLayout = 8,
    /* Both protocols: hierarchical summation order for nodes of this many
     * consecutive ranks: each node's partial is summed in binary32 in rank
     * order, then the partials in node order, then rounded once -- the result
     * of a two-level all-reduce that reduces inside each node first and across
     * nodes second ("SGLang 中的 MSCCL++ All-Reduce 基准测试与推理集成指南",
     * section 4.4: multi-node algorithms for TP = 16 / 32).  0 (default), 1
     * or >= nranks: the flat order 0..R-1.  A value in between must divide
     * nranks (else arInvalidUsage).  The two ablations keep the flat order:
     * with arOptHBStaged, HB returns arUnsupported, and with the sequenced LL
     * flag scheme, LL does (arProtoAuto then runs HB). */
    arOptNodeRanks = 9,
    /* LL: packet width in bytes.  8: a 4-byte payload next to a 4-byte flag;
     * 16: two such pairs, written and read as one 16-byte access (half the
     * memory instructions per payload byte).  0 (default): the width the
     * tuner chose for the message size, else the built-in default's for the
     * rank count and size (16 bytes from 256 KiB per rank up to 8 ranks and
     * from 128 KiB above 16 ranks; 8 bytes otherwise).  16 needs the communicator's
     * packet memory below 4 GiB (maxRanks * maxLLBytesPerRank * 2), else
     * setting it returns arUnsupported. */
    arOptLLPacketBytes = 10,
    /* HB: 1 = the staged two-shot, an ablation of the fused default: the
     * reduce-scatter writes each reduced chunk to its owner rank's output
     * only, a kernel boundary stands for the synchronisation between the
     * shots (the HB protocol synchronises rarely, "MSCCL++：让 GPU 通信像 CUDA
     * 一样可编程", "MemoryChannel"), and the all-gather copies each chunk from
     * its owner to the other outputs.  Same result bits; 2 * bytes per rank
     * more traffic and one more launch.  Launch shape from arOptHBThreads /
     * arOptHBBlocks or the defaults, never the tuned table.  With
     * arOptNodeRanks set, HB calls return arUnsupported.  0 (default): fused. */
    arOptHBStaged = 11,
    /* LL: how a packet left by an earlier call is kept from looking ready.
     * 0 (default): the reader zeroes every packet it has consumed, so packet
     * memory is zero between calls (one extra store per packet).  1: every
     * 512-byte group of a rank's packets carries a 32-bit sequence number in a
     * table owned by the communicator; producers flag packets with the
     * group's next number and the group's reader advances it, so nothing is
     * cleared.  An ablation: slower on MI355X at every LL size, since each
     * producer reads the table before it can store.  Both give the same
     * results and may be mixed from call to call.  With 1, the launch shape
     * comes from the LL options or the defaults, never the tuned table. */
    arOptLLFlagScheme = 12,
    /* Test hook: the value arCommReset writes to every sequence-table entry
     * (0 .. 0xFFFFFFFF; default 0), to exercise the sequence numbers' wrap.
     * Takes effect at the next arCommReset. */
    arOptDebugSeqStart = 13,
    /* arCommTune's timing method.  0 (default): each candidate replays on
     * unchanged inputs, which stay in the last-level cache between calls, as
     * the benchmark's graph replays do.  1: before each timed call a copy-like
     * kernel rewrites the inputs (every 16-byte vector of each rank's
     * message), as when every step of a model produces new inputs; the
     * rewrites' own time, measured alone, is subtracted.  On MI355X this
     * changes the HB access policy that wins from a few MiB per rank up. */
    arOptTuneFreshInputs = 14
} arOption_t;

/* Create a communicator on `device` for groups of up to `maxRanks` (1..32)
 * simulated ranks and LL messages of up to `maxLLBytesPerRank` bytes per rank.
 * It owns device memory for the LL packets (2 * maxRanks * maxLLBytesPerRank
 * bytes, each rank's share rounded up to 512 bytes: packets are half payload,
 * half flags, at either width), a sequence table of 1/128 of that size (see
 * arOptLLFlagScheme) and a word that records an asynchronous error.  maxLLBytesPerRank
 * may be 0 (HB only).  Allocates with hipMalloc, so it must not be called
 * while a stream is being captured.  The caller's current device is left
 * unchanged.
 * Returns arInvalidArgument for a NULL `comm` or out-of-range sizes,
 * arHipError if the device or memory is not available. */
arResult_t arCommCreate(arComm_t *comm, int device, int maxRanks, size_t maxLLBytesPerRank);

/* Free the communicator.  Work that uses it must have finished. */
arResult_t arCommDestroy(arComm_t comm);

/* Enqueue, on `stream`, a kernel that clears the LL packets, the sequence
 * table (to arOptDebugSeqStart, 0 by default) and the asynchronous error, so
 * that the communicator can be used again after a timeout (an LL call that
 * timed out may leave packets set; LL results are undefined until the reset).
 * No allocation and no memset node: safe to capture in a graph. */
arResult_t arCommReset(arComm_t comm, arStream_t stream);

/* Read the asynchronous error recorded by earlier kernels: arSuccess or
 * arTimeout.  Synchronises the device first.  The error stays set until
 * arCommReset. */
arResult_t arCommGetAsyncError(arComm_t comm, arResult_t *asyncError);

/* Set or read one option (arOption_t) of the communicator.  Values outside an
 * option's range give arInvalidArgument. */
arResult_t arCommSetOption(arComm_t comm, arOption_t option, int64_t value);
arResult_t arCommGetOption(arComm_t comm, arOption_t option, int64_t *value);

/* Measure launch shapes and keep the fastest, per message size -- the
 * start-up tuning of SGLang's MSCCL++ integration ("SGLang 中的 MSCCL++
 * All-Reduce 基准测试与推理集成指南", blog.gitcode.com, section 4.4: every
 * power-of-two size timed over (workgroups, threads per workgroup) candidates,
 * the best kept for the life of the process).
 *
 * For `dtype` and `nranks`, every power-of-two size from 512 bytes up to
 * maxBytesPerRank per rank (the last bucket at maxBytesPerRank itself) is
 * timed with each protocol the communicator can run at that size, in place
 * and out of place (the two favour different shapes), over the built-in
 * default shape and a fixed set of candidates; a candidate wins only if it is
 * more than 3 % faster than the best before it, and the winner and its time
 * are stored in the communicator.  Later calls of that dtype and rank count
 * use the stored shape of their size bucket (the message size rounded up to a
 * power of two) and mode (in place: recvbufs[r] == sendbufs[r] for every
 * rank) unless arOptLLThreads/arOptLLBlocksPerRank (LL) or arOptHBThreads/
 * arOptHBBlocks (HB), arOptLLPacketBytes or arOptLLFlagScheme are set;
 * arProtoAuto then picks the faster protocol.  LL candidates cover both
 * packet widths, in the default flag scheme; HB candidates both access
 * policies unless arOptHBNonTemporal fixes one.
 * Tuning again overwrites the table; sizes never tuned use built-in defaults.
 *
 * Each candidate is timed the way latency-sensitive callers run the library:
 * its calls captured into a HIP graph on a private stream of the tuner, and
 * the graph replayed (eager launches would time the host's launch rate at
 * small sizes); with arOptTuneFreshInputs = 1, each call right after a
 * rewrite of its inputs, the rewrites' time subtracted.  Allocates two scratch planes of nranks * maxBytesPerRank
 * bytes for the duration, waits for `stream` first and synchronises the
 * device at the end: never call it while a stream is being captured.
 * Returns arInvalidArgument for a NULL comm or maxBytesPerRank outside
 * 512 B .. 16 GiB, arUnsupported for a dtype or rank
 * count arAllReduce would reject, arInvalidUsage if the communicator is not on
 * the current device, arHipError if memory or a launch fails, arTimeout if an
 * LL wait ran out during tuning (then reset the communicator). */
arResult_t arCommTune(arComm_t comm, arDataType_t dtype, int nranks, size_t maxBytesPerRank,
                      arStream_t stream);

/* One entry of the tuned table. */
typedef struct {
    int tuned;        /* 0: this size was never tuned (the rest is 0) */
    int threads;      /* threads per workgroup that won; 0 with blocks 0: the default shape */
    int blocks;       /* workgroups that won (HB: the grid; LL: per rank) */
    int packetBytes;  /* LL: the packet width that won, 8 or 16; HB: 0 */
    int nonTemporal;  /* HB: 1 if non-temporal accesses won, 0 if cached ones; LL: 0 */
    float us;         /* time per call measured for it, in microseconds */
} arTunedShape_t;

/* The tuned entry for (dtype, nranks, protocol LL or HB) at a message of
 * bytesPerRank bytes, in place (inPlace = 1) or out of place (inPlace = 0),
 * copied to *shape.  Returns arInvalidArgument for NULL pointers or
 * out-of-range arguments. */
arResult_t arCommGetTunedShape(arComm_t comm, arDataType_t dtype, int nranks,
                               arProtocol_t protocol, size_t bytesPerRank, int inPlace,
                               arTunedShape_t *shape);

/* The sum all-reduce.
 *
 *  sendbufs  host array of `nranks` device pointers; sendbufs[r] holds rank
 *            r's `count` elements, contiguous.  Read only during the call.
 *  recvbufs  host array of `nranks` device pointers for the results, laid
 *            out like sendbufs.  recvbufs[r] == sendbufs[r] for a rank means
 *            in place; the result is then computed from the values the
 *            buffers held when the kernel started.
 *  count     elements per rank.  0 returns arSuccess and enqueues nothing.
 *  dtype     arBfloat16, arFloat16 or arFloat32 (else arUnsupported).
 *  op        arSum only (else arUnsupported).
 *  nranks    1..32 (else arUnsupported); 1 is a copy.
 *  protocol  arProtoLL, arProtoHB or arProtoAuto (else arInvalidArgument).
 *  comm      a communicator on the current device.
 *  stream    the stream to enqueue on.
 *
 * Rules (arInvalidArgument when broken): no NULL pointer; every pointer
 * 16-byte aligned; the 2*nranks byte ranges do not overlap except that a
 * receive buffer may coincide exactly with the same rank's send buffer, and
 * send buffers may overlap one another (they are only read).
 * LL also needs nranks <= the communicator's maxRanks and count * element
 * size <= its maxLLBytesPerRank (arInvalidUsage otherwise); arProtoAuto only
 * picks LL where it can run.  With a hierarchical order set (arOptNodeRanks),
 * nranks must be a multiple of the node size (arInvalidUsage otherwise), and
 * the staged HB form and the sequenced LL scheme return arUnsupported.
 *
 * The call only enqueues work and returns; the buffers belong to the caller
 * and must stay valid until the work has run (for a captured graph, as long
 * as the graph is replayed).  Nothing is allocated or synchronised, so calls
 * can be captured into a HIP graph.  Validation makes no HIP call, so every
 * argument error is reported without touching the device. */
arResult_t arAllReduce(const void *const *sendbufs, void *const *recvbufs, size_t count,
                       arDataType_t dtype, arRedOp_t op, int nranks, arProtocol_t protocol,
                       arComm_t comm, arStream_t stream);

/* Static description of a result code. */
const char *arGetErrorString(arResult_t result);

/* AR_VERSION of the built library. */
int arGetVersion(void);

#ifdef __cplusplus
}
#endif

#endif /* AR_ALLREDUCE_H */
