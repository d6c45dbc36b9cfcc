// Disk tier of the layer store: the records of the layers that do not stay
// in pinned host memory live in one file and reach the device slots through
// pinned staging buffers (page "Can You Fine-Tune Llama 3.1 8B on a 4GB
// GPU? ...", section "How Soup's layer streaming actually works", item 2, and
// its FAQ on using an SSD: the frozen store may spill to NVMe when host
// memory cannot hold it, at the cost of another bandwidth bound).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <condition_variable>
#include <deque>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

// Record slots of kDiskAlign-padded size, file index i = layer - first disk layer.
constexpr int64_t kDiskAlign = 4096;

// Reads are buffered preads straight into the pinned staging buffers (direct
// I/O cannot target driver-mapped pinned pages: the kernel refuses to pin them
// again), and each record's pages are dropped from the page cache after the
// read, so every read of a disk layer comes from the device rather than from
// host memory.

class DiskFile {
 public:
  ~DiskFile() { close_and_unlink(); }
  // Creates (truncates) `path` for n records of record_bytes.
  int open(const std::string& path, int64_t record_bytes, int n, std::string* why);
  // 0 or -errno.  write: record idx from any buffer.  read_any: its bytes into
  // any buffer.  read_from_device: the same in `parts` concurrent preads, then
  // drops the record's pages from the page cache.  flush_and_drop: writes
  // the file back and drops all of its cached pages.
  int write(int idx, const uint8_t* rec) const;
  int read_any(int idx, uint8_t* buf) const;
  int read_from_device(int idx, uint8_t* buf, int parts) const;
  int flush_and_drop() const;
  void close_and_unlink();
  int64_t padded() const { return padded_; }
  int64_t record_bytes() const { return bytes_; }
  bool is_open() const { return fd_ >= 0; }

 private:
  int fd_ = -1, n_ = 0;
  int64_t bytes_ = 0, padded_ = 0;
  std::string path_;
};

// Session-side read-ahead over a DiskFile: a thread fills nbuf pinned staging
// buffers with records, the next disk layer in the sweep's direction read
// ahead of the request for it.  take() blocks until the requested record is
// in a buffer; after_copy() records the copy that drains the buffer, and the
// thread waits for that copy before it refills the buffer.
class DiskReader {
 public:
  struct Stats { int64_t reads = 0, bytes = 0; double read_ms = 0, wait_ms = 0; };
  ~DiskReader();
  // first: index of the first disk layer; n_layers: all layers.
  int init(const DiskFile* f, int first, int n_layers, int nbuf, std::string* why);
  // Staging buffer holding `layer` (nullptr on a read error, see error());
  // dir = +1 / -1: the sweep's direction, for the read-ahead.
  const uint8_t* take(int layer, int dir, int* buf);
  // The copy on `stream` that drains buffer `buf` has been enqueued.
  int after_copy(int buf, hipStream_t stream);
  Stats stats();
  void reset_stats();
  const std::string& error() const { return err_; }

 private:
  enum State { FREE, QUEUED, READING, READY, TAKEN };
  struct Buf {
    uint8_t* p = nullptr;
    int layer = -1;
    State state = FREE;
    hipEvent_t copied = nullptr;
    bool copy_pending = false;
    int rc = 0;
  };
  int claim(int layer, bool may_wait, std::unique_lock<std::mutex>& lk);
  void run();

  const DiskFile* f_ = nullptr;
  int first_ = 0, n_layers_ = 0;
  std::vector<Buf> bufs_;
  std::deque<int> jobs_;
  std::mutex mu_;
  std::condition_variable cv_;
  std::thread th_;
  bool stop_ = false;
  Stats st_;
  std::string err_;
};
