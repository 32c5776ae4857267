// Streaming of finished step tables to the device (the rebuild pipeline:
// ZeroGR summary, "Does it actually work better?", rebuilding paragraph: the
// new index is built on the CPU in parallel chunks whose final positions are
// computed in advance, and streamed to the GPU in batches through two
// alternating buffers, without taking GPU time from live traffic).
//
// A host thread of its own takes the steps in the order the builder finishes
// them; each array is copied in batches through two pinned staging buffers on
// a copy stream of its own, so that the host fills one buffer while the other
// is in flight, and the builder works on the next step meanwhile.  Only
// copies are enqueued (no kernels), on a stream of default priority.
#include <hip/hip_runtime.h>

#include <cstring>

#include "cb_internal.h"

namespace cb {

namespace {
constexpr size_t kStageBytes = size_t(32) << 20;  // per staging buffer
}

StepUploader::StepUploader(cb_index* idx) : idx_(idx) {}

StepUploader::~StepUploader() { (void)finish(); }

void StepUploader::fail(const std::string& m) {
    if (status_ == CB_OK) {
        status_ = CB_EHIP;
        msg_ = m;
    }
}

cb_status StepUploader::start() {
    DeviceGuard g(idx_->device);
    if (!g.ok) {
        set_error("cb_build_index: cannot select device " + std::to_string(idx_->device));
        return CB_EHIP;
    }
    hipError_t e = hipStreamCreateWithFlags(&stream_, hipStreamNonBlocking);
    for (int i = 0; i < 2 && e == hipSuccess; ++i) {
        e = hipHostMalloc(&stage_[i], kStageBytes, hipHostMallocDefault);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&ev_[i], hipEventDisableTiming);
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        release();
        set_error(std::string("cb_build_index: upload set-up failed: ") + hipGetErrorString(e));
        return CB_EHIP;
    }
    thread_ = std::thread([this] { run(); });
    started_ = true;
    return CB_OK;
}

void StepUploader::push(int t) {
    {
        std::lock_guard<std::mutex> lk(mu_);
        queue_.push_back(t);
    }
    cv_.notify_one();
}

cb_status StepUploader::finish() {
    if (started_) {
        {
            std::lock_guard<std::mutex> lk(mu_);
            closed_ = true;
        }
        cv_.notify_one();
        thread_.join();
        started_ = false;
    }
    release();
    if (status_ != CB_OK) set_error(msg_);
    return status_;
}

void StepUploader::release() {
    DeviceGuard g(idx_->device);
    for (int i = 0; i < 2; ++i) {
        if (ev_[i]) (void)hipEventDestroy(ev_[i]);
        if (stage_[i]) (void)hipHostFree(stage_[i]);
        ev_[i] = nullptr;
        stage_[i] = nullptr;
    }
    if (stream_) (void)hipStreamDestroy(stream_);
    stream_ = nullptr;
}

// Copy n bytes from host src to device dst in batches through the staging
// buffers: a buffer is refilled only once the copy that last read it is done.
bool StepUploader::stream_copy(void* dst, const void* src, size_t n) {
    const unsigned char* s = static_cast<const unsigned char*>(src);
    unsigned char* d = static_cast<unsigned char*>(dst);
    for (size_t off = 0; off < n; off += kStageBytes) {
        const size_t m = std::min(kStageBytes, n - off);
        hipError_t e = hipEventSynchronize(ev_[cur_]);
        if (e == hipSuccess) {
            std::memcpy(stage_[cur_], s + off, m);
            e = hipMemcpyAsync(d + off, stage_[cur_], m, hipMemcpyHostToDevice, stream_);
        }
        if (e == hipSuccess) e = hipEventRecord(ev_[cur_], stream_);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            fail(std::string("cb_build_index: upload: ") + hipGetErrorString(e));
            return false;
        }
        cur_ ^= 1;
    }
    return true;
}

template <class T>
bool StepUploader::upload_array(std::vector<T>& host, T** dev, const char* what) {
    *dev = nullptr;
    if (host.empty()) return true;
    const hipError_t e = hipMalloc(reinterpret_cast<void**>(dev), host.size() * sizeof(T));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *dev = nullptr;
        if (status_ == CB_OK) {
            status_ = CB_ENOMEM;
            msg_ = std::string("device allocation failed: ") + what;
        }
        return false;
    }
    return stream_copy(*dev, host.data(), host.size() * sizeof(T));
}

void StepUploader::run() {
    if (hipSetDevice(idx_->device) != hipSuccess) {
        (void)hipGetLastError();
        fail("cb_build_index: cannot select the device in the upload thread");
    }
    for (;;) {
        int t;
        {
            std::unique_lock<std::mutex> lk(mu_);
            cv_.wait(lk, [this] { return closed_ || !queue_.empty(); });
            if (queue_.empty()) break;
            t = queue_.front();
            queue_.pop_front();
        }
        if (status_ != CB_OK) continue;  // drain the queue after a failure
        StepTable& T = idx_->steps[(size_t)t];
        bool ok = upload_array(T.row_ptr, &T.d_row_ptr, "row_ptr") && upload_array(T.tok, &T.d_tok, "tokens") &&
                  upload_array(T.bits, &T.d_bits, "bitmap") && upload_array(T.rank, &T.d_rank, "rank directory") &&
                  upload_array(T.tok0, &T.d_tok0, "first tokens");
        // the host arrays may go once their last batches are in flight and done
        if (ok && hipStreamSynchronize(stream_) != hipSuccess) {
            (void)hipGetLastError();
            fail("cb_build_index: upload: stream synchronisation failed");
            ok = false;
        }
        if (ok) {
            std::vector<uint32_t>().swap(T.row_ptr);
            std::vector<uint16_t>().swap(T.tok);
            std::vector<uint32_t>().swap(T.bits);
            std::vector<uint16_t>().swap(T.rank);
            std::vector<uint16_t>().swap(T.tok0);
        }
    }
}

}  // namespace cb
